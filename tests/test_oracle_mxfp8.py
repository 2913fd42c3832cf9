"""Pins of the oracle's MXFP8 activation rounding (E4M3 elements, one E8M0
scale per 32 values; OCP Microscaling Formats spec v1.0, sections 5.3.3
and 6.3) against facts that do not come from the oracle's own code: the
format's named values, its ordering, a brute-force nearest-value search over
every code, and the spec's scale rule on exact powers of two."""
import numpy as np
import pytest

import oracle
import synth

FINITE = [c for c in range(256) if (c & 0x7F) != 0x7F]


def _values():
    return {c: oracle.e4m3_value(c) for c in FINITE}


def test_e4m3_named_values():
    # OCP 8-bit floating point formats: E4M3 bias 7, no infinities, S.1111.111 is NaN
    v = oracle.e4m3_value
    assert v(0x38) == 1.0
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0          # largest normal 1.75 * 2^8
    assert v(0x08) == 2.0 ** -6                              # smallest normal
    assert v(0x07) == 0.875 * 2.0 ** -6                      # largest subnormal
    assert v(0x01) == 2.0 ** -9                              # smallest subnormal
    assert v(0x00) == 0.0 and v(0x80) == 0.0
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    assert v(0x38, 130) == 8.0 and v(0x38, 120) == 2.0 ** -7  # E8M0 scale 2^(s-127)


def test_e4m3_ordering_and_grid():
    vals = _values()
    pos = [vals[c] for c in range(0x00, 0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:])), "codes 0x00..0x7E must increase"
    assert all(vals[c | 0x80] == -vals[c] for c in range(0x7F))
    # eight values per binade, evenly spaced; the subnormal step equals the first binade's
    for e in range(1, 16):
        b = [vals[(e << 3) | m] for m in range(8) if ((e << 3) | m) != 0x7F]
        steps = np.diff(b)
        assert np.all(steps == steps[0]) and steps[0] == 2.0 ** (e - 7 - 3)
    assert vals[0x01] - vals[0x00] == vals[0x09] - vals[0x08]
    # every value is exact in bf16 (8 significant bits, wide exponent)
    for x in pos:
        f = np.float32(x)
        assert float(synth.bf16_to_f32(synth.bf16_bits(np.array([f])))[0]) == x


def _nearest_code(q, vals):
    """Brute force: the finite code nearest to q (ties to the even mantissa),
    magnitudes beyond 448 saturated."""
    if abs(q) >= 448.0:
        return 0x7E | (0x80 if q < 0 else 0)
    best, bd = None, None
    for c in FINITE:
        d = abs(vals[c] - q)
        if bd is None or d < bd or (d == bd and (c & 1) == 0 and (best & 1) == 1):
            best, bd = c, d
    return best


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_quantize_is_nearest_value(seed):
    rng = np.random.default_rng(seed)
    vals = _values()
    blocks = []
    for kind in range(6):
        if kind == 0:
            b = rng.standard_normal(32)
        elif kind == 1:
            b = rng.standard_normal(32) * 2.0 ** rng.integers(-20, 20)
        elif kind == 2:   # wide dynamic range inside a block: subnormal elements
            b = rng.standard_normal(32) * 2.0 ** rng.integers(-14, 2, size=32)
        elif kind == 3:   # exact ties between neighbouring codes
            sc = 2.0 ** rng.integers(-6, 6)
            c = rng.choice(np.arange(0x09, 0x76), 32)
            b = (np.array([vals[int(x)] for x in c]) + np.array([vals[int(x) + 1] for x in c])) / 2 * sc
            b[0] = 440.0 * sc  # sets the scale to sc
        elif kind == 4:   # elements that saturate (scaled max in (448, 512))
            b = rng.uniform(-1, 1, 32)
            b[5] = 0.99
        else:
            b = np.zeros(32)
            b[3] = -2.0 ** -30
        blocks.append(b)
    v = np.concatenate(blocks)
    codes, scales = oracle.mxfp8_quantize(v)
    for i, b in enumerate(blocks):
        amax = np.abs(b).max()
        e = int(np.floor(np.log2(amax)))
        assert 2.0 ** e <= amax < 2.0 ** (e + 1)
        assert scales[i] == e - 8 + 127
        for j in range(32):
            q = b[j] / 2.0 ** (e - 8)
            want = _nearest_code(q, vals)
            got = int(codes[i * 32 + j])
            assert got == want or (vals[got] == vals[want] == 0.0), (i, j, q, got, want)


def test_scale_rule_and_zero_block():
    for e in (-10, -1, 0, 3, 9):
        for amax in (2.0 ** e, 2.0 ** (e + 1) * (1 - 2 ** -40)):
            v = np.zeros(32)
            v[7] = amax
            codes, scales = oracle.mxfp8_quantize(v)
            assert scales[0] == e - 8 + 127
    codes, scales = oracle.mxfp8_quantize(np.zeros(64))
    assert (codes == 0).all() and (scales == 0).all()


def test_round_idempotent_and_error_bound():
    rng = np.random.default_rng(7)
    v = rng.standard_normal(32 * 200) * 2.0 ** rng.integers(-8, 8, size=32 * 200)
    r = oracle.mxfp8_round(v)
    assert np.array_equal(oracle.mxfp8_round(r), r)
    vb = v.reshape(-1, 32)
    rb = r.reshape(-1, 32)
    X = 2.0 ** (np.floor(np.log2(np.abs(vb).max(1))) - 8)[:, None]
    q = np.abs(vb) / X
    normal = (q >= 2.0 ** -6) & (q <= 448)
    # half of the 2^-3 relative spacing of a binade
    assert np.all(np.abs(rb - vb)[normal] <= 2.0 ** -4 * 2.0 ** np.floor(np.log2(np.abs(vb)[normal])))
    sub = q < 2.0 ** -6
    assert np.all(np.abs(rb - vb)[sub] <= (2.0 ** -10 * X * np.ones_like(vb))[sub])
    sat = q > 448
    assert np.all(np.abs(rb)[sat] == (448 * X * np.ones_like(vb))[sat])


def _one_hot_oai_case(quant):
    """gpt-oss expert with one-hot gate/up rows: gate row f reads input 2f,
    up row f reads input 2f + 1, so the activation is a closed form of two
    inputs; down is the identity on the first F outputs."""
    H, F, E, k = 64, 32, 2, 1
    c = synth.make_case("gptoss20b_bf16", T=3, E=E, H=H, F=F, k=k)
    c.act_quant = "mxfp8" if quant else "none"
    gu = np.zeros((E, 2 * F, H), np.float32)
    for f in range(F):
        gu[:, 2 * f, 2 * f] = 1.0
        gu[:, 2 * f + 1, 2 * f + 1] = 1.0
    dn = np.zeros((E, H, F), np.float32)
    for f in range(F):
        dn[:, f, f] = 1.0
    c.t["gate_up_w"] = synth.bf16_bits(gu)
    c.t["down_w"] = synth.bf16_bits(dn)
    c.t["gate_up_b"] = np.zeros((E, 2 * F), np.uint16)
    c.t["down_b"] = np.zeros((E, H), np.uint16)
    return c


def _oai(g, u, alpha=1.702, lim=7.0):
    g = np.minimum(g, lim)
    u = np.clip(u, -lim, lim)
    return (u + 1.0) * g / (1.0 + np.exp(-alpha * g))


def test_layer_rounds_routed_inputs():
    """Closed form of a one-hot layer with and without MXFP8 inputs: the
    expert sees x rounded to MXFP8 and the down product sees h rounded."""
    for quant in (False, True):
        c = _one_hot_oai_case(quant)
        out, idx, wt, _ = oracle.Layer(c).forward()
        x = synth.bf16_to_f32(c.t["x"]).astype(np.float64)
        for t in range(c.T):
            xi = oracle.mxfp8_round(x[t]) if quant else x[t]
            h = _oai(xi[0::2][:c.F], xi[1::2][:c.F])
            hq = oracle.mxfp8_round(h) if quant else h
            want = np.zeros(c.H)
            want[:c.F] = hq * float(wt[t, 0])
            np.testing.assert_allclose(out[t], want, rtol=1e-6, atol=1e-6)
    # the rounding is visible: some token's output changes
    a = oracle.Layer(_one_hot_oai_case(False)).forward()[0]
    b = oracle.Layer(_one_hot_oai_case(True)).forward()[0]
    assert np.abs(a - b).max() > 0


def test_quantized_layer_differs_from_plain_layer():
    """MXFP8 inputs change the MXFP4 layer's output (finite, nonzero
    difference).  Its size depends on the weights: on these synthetic MXFP4
    weights, whose block scales span 2^-9..2^3, a few blocks dominate each
    output and the difference is ~17% of max|out|, which is why the GPU's
    MXFP8 path is compared with this oracle mode, not with the plain one."""
    c = synth.make_case("gptoss20b_mxfp4", T=4, E=4, H=256, F=128, k=2)
    plain = oracle.Layer(c).forward()[0]
    c.act_quant = "mxfp8"
    quant = oracle.Layer(c).forward()[0]
    assert np.all(np.isfinite(quant))
    err = np.abs(quant - plain).max() / np.abs(plain).max()
    assert 0 < err < 1

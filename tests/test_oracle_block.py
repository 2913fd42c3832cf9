"""Pins of the oracle's decoder-block prologue and epilogue: the RMSNorm in
front of the layer and the residual add behind it ("qwen35moe - Forward-Pass
Design (Pantheon port)", section "Block scaffold"; "Phase 19: MoE -
gpt-oss-20b", section 2 RMSNorm and decoder layer; "qwen35moe CPU-reference
golden vectors", Kernel 3 for the norm's formula).

The norm is pinned to hand-worked values of the formula, closed forms
(constant rows, unit RMS, invariance under power-of-two scaling with eps = 0,
where a dropped square root or a sum in place of the mean would fail) and
the bf16 storage rounding of exactly representable results; the block to
the definition out = r + layer(norm(r)) with the layer's own output."""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rmsnorm_worked.json")


def _norm(x, w, eps, dtype="f32"):
    x = np.asarray(x, np.float32)
    w = np.asarray(w, np.float32)
    if dtype == "bf16":
        return oracle.rmsnorm(synth.bf16_bits(x), synth.bf16_bits(w), eps, "bf16")
    return oracle.rmsnorm(x, w, eps, "f32")


@pytest.mark.parametrize("i", range(5))
def test_rmsnorm_hand_worked(i):
    case = json.load(open(GOLDEN))["cases"][i]
    got = _norm(np.array([case["x"]]), case["w"], case["eps"])[0]
    np.testing.assert_allclose(got, case["y"], rtol=1e-7, atol=0)


def test_rmsnorm_constant_rows_closed_form():
    H = 64
    for c in (0.25, -3.0, 1000.0):
        for eps in (0.0, 1e-6, 0.5):
            got = _norm(np.full((1, H), c), np.ones(H), eps)[0]
            want = np.sign(c) / np.sqrt(1.0 + eps / (c * c))
            np.testing.assert_allclose(got, want, rtol=1e-7)


def test_rmsnorm_unit_rms_and_weight():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 320)).astype(np.float32) * np.float32(7.0)
    y = _norm(x, np.ones(320), 0.0).astype(np.float64)
    np.testing.assert_allclose((y * y).mean(1), 1.0, rtol=1e-6)
    w = (1.0 + 0.1 * rng.standard_normal(320)).astype(np.float32)
    yw = _norm(x, w, 0.0).astype(np.float64)
    np.testing.assert_allclose(yw, y * w, rtol=1e-6)        # the weight scales each column


def test_rmsnorm_power_of_two_scaling_invariant():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 256)).astype(np.float32)
    w = (1.0 + 0.1 * rng.standard_normal(256)).astype(np.float32)
    base = _norm(x, w, 0.0)
    for k in (-20, -3, 5, 30):
        assert np.array_equal(_norm(x * np.float32(2.0 ** k), w, 0.0), base)
    # bf16 storage too
    bb = _norm(x, w, 0.0, "bf16")
    assert np.array_equal(_norm(x * np.float32(8.0), w, 0.0, "bf16"), bb)


def test_rmsnorm_bf16_storage_rounding():
    # a constant row with eps = 0 normalises to exactly +-1 (bf16 0x3F80 / 0xBF80)
    assert np.all(_norm(np.full((1, 32), 5.0), np.ones(32), 0.0, "bf16") == 0x3F80)
    assert np.all(_norm(np.full((1, 32), -0.125), np.ones(32), 0.0, "bf16") == 0xBF80)
    # y = w / 2 for x = 1, eps = 3: every bf16 w halves exactly
    w = synth.bf16_to_f32(synth.bf16_bits(np.linspace(0.5, 2.0, 32).astype(np.float32)))
    got = _norm(np.ones((1, 32)), w, 3.0, "bf16")[0]
    assert np.array_equal(synth.bf16_to_f32(got), (w / 2).astype(np.float32))


@pytest.mark.parametrize("name,T", [("tiny_fp32", 8), ("qwen35moe_decode", 3), ("gptoss20b_bf16", 2)])
def test_block_is_residual_plus_layer_of_normalised_input(name, T):
    over = {} if name == "tiny_fp32" else dict(E=16, H=256, F=128, k=4) if name.startswith("gptoss") else \
        dict(E=16, H=256, F=128, Fs=128, k=4)
    c = synth.add_block_inputs(synth.make_case(name, T=T, **over))
    L = oracle.Layer(c)
    out, xn, idx, wt, sg = L.block_forward()
    # the layer run on the normalised rows
    c.t["x"] = xn
    plain, idx2, _, _ = oracle.Layer(c).forward()
    assert np.array_equal(idx, idx2)
    r = synth.bf16_to_f32(c.t["resid"]) if c.x_dtype == "bf16" else c.t["resid"]
    np.testing.assert_allclose(out.astype(np.float64) - plain, r, atol=4 * np.abs(out).max() * 2.0 ** -24)
    # the residual is the un-normalised input, not the normalised one
    xs = synth.bf16_to_f32(xn) if c.x_dtype == "bf16" else xn
    assert np.abs((out.astype(np.float64) - plain) - xs).max() > 0.1


def test_block_inputs_have_per_token_rms():
    c = synth.add_block_inputs(synth.make_case("qwen35moe_decode", T=8))
    r = synth.bf16_to_f32(c.t["resid"]).astype(np.float64)
    rms = np.sqrt((r * r).mean(1))
    assert rms.max() / rms.min() > 4.0          # tokens at different scales
    assert c.norm_eps == 1e-6
    g = synth.add_block_inputs(synth.make_case("gptoss20b_bf16", T=2, only=("x",)))
    assert g.norm_eps == 1e-5

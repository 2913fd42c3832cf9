"""GPU layer inside its pre-norm decoder block (moe_forward_prenorm):
RMSNorm of the residual stream in front, residual add behind, against the
oracle's block on the same seeded inputs.

* normalised rows: bf16 outputs bit-equal to the oracle's for >= 99.9% of
  elements and never more than one bf16 step apart (the GPU sums squares in
  fp32 in its own order, so a value next to a rounding boundary may round
  the other way); fp32 outputs within 2e-6 relative;
* the layer part out - resid: the layer tolerance of the weights' dtype
  (max|err| <= tol * max|ref|) on every sampled token; one routed
  differently (only inside the rounding bound of its logits) is compared
  with the oracle's block on the GPU's picks;
* the residual add: bit-equal to fp32(resid + moe_forward(xn)) run on the
  GPU's own normalised rows (for up to 64 tokens the router-product kernel
  normalises on the fly, so this also checks that its logits equal the
  plain router's on the rows it wrote)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_ffn_router_amd as moe
import synth
from tests._gpu import config_of, device_weights, to_torch
from tests._parity import assert_normwise, cached_case, check_layer_output, log, tol_of

pytestmark = pytest.mark.gpu

BLOCKS = [
    ("tiny_fp32", 8, None, {}),
    ("qwen35moe_decode", 8, None, {}),                                    # decode shape
    ("qwen35moe_decode", 200, None, dict(E=16, H=256, F=192, Fs=128, k=4)),  # MFMA tiles
    ("qwen35moe_prefill_zipf", 4096, 40, {}),                             # prefill shape, drawn logits
    ("gptoss20b_bf16", 16, None, dict(E=8, H=320, F=192, k=2)),           # 40 pieces per row (ragged lanes)
    ("gptoss20b_bf16", 2048, 20, {}),
    ("gptoss20b_mxfp4", 16, None, {}),                                    # decode shape
    ("gptoss20b_mxfp4", 150, None, dict(E=8, H=320, F=192, k=2)),
    ("qwen35moe_decode", 64, 16, {}),                                     # largest batch normalised in the router
    ("qwen35moe_decode", 65, 16, {}),                                     # smallest with its own norm launch
    ("gptoss20b_bf16", 64, None, dict(E=8, H=320, F=192, k=2)),           # 8 router waves write 64 rows
    ("qwen35moe_prefill_zipf", 8, None, {}),                              # drawn logits at decode size: RMSNorm launch
    ("tiny_fp32", 100, None, {}),                                         # fp32 rows past 64 tokens
    ("qwen35moe_decode", 13, None, dict(E=8, H=4096, F=128, Fs=128, k=2)),  # widest rows normalised in the router
    ("qwen35moe_decode", 6, None, dict(E=8, H=3072, F=128, Fs=128, k=2)),   # 6 pieces per lane
]


def test_prenorm_block_mxfp8_inputs():
    # the MX MFMA path reads the normalised rows rounded to MXFP8
    case = _case("gptoss20b_mxfp4", 150, dict(E=8, H=320, F=192, k=2))
    case.act_quant = "mxfp8"
    cfg, w, out, xn, idx, ws = _run(case)
    tokens = np.arange(case.T, dtype=np.int32)
    rel = _check_block(case, tokens, idx, out, 3e-2, "mxfp8 block layer part")
    log("  mxfp8 block: max|err|/max|ref| = %.3e" % rel)


def _check_block(case, tokens, idx, out, tol, what):
    """The layer part (out - resid) of the sampled tokens against the
    oracle's block.  The router reads the normalised rows, whose bf16
    elements may sit one step from the oracle's, so a token may route
    differently only inside the rounding bound of its logits; it is then
    compared with the oracle's block on the GPU's picks.  Drawn logits are
    the same on both sides, so there every token must route alike."""
    L = oracle.Layer(case)
    lg = case.t.get("logits") if case.drawn_logits else None
    r_out, r_xn, r_idx, _, _ = L.block_forward(tokens=tokens, logits=lg)
    r64 = _f64(case.t["resid"], case.x_dtype)
    ref_lg = case.t["logits"][tokens] if case.drawn_logits else \
        oracle.Layer(_with_x(case, r_xn)).router_logits()[tokens]
    redo = lambda gi, tk: L.block_forward(tokens=tk, logits=lg, idx=gi)[0] - r64
    return check_layer_output(case, tokens, idx.cpu().numpy(), out.cpu().numpy().astype(np.float64) - r64,
                              r_out.astype(np.float64) - r64, r_idx, ref_lg, redo, tol, what,
                              exact_routing=case.drawn_logits, x=r_xn)


def _with_x(case, x):
    c = synth.Case(case.name, case.T, case.H, case.E, case.k, case.F, case.Fs, case.gating, case.norm_topk_prob,
                   case.weights_scale, case.act, case.alpha, case.limit, case.x_dtype, case.w_dtype,
                   case.router_dtype)
    c.t = dict(case.t)
    c.t["x"] = x
    return c


def _ids(p):
    name, T, s, over = p
    return "%s-T%d%s" % (name, T, "-" + "-".join("%s%d" % kv for kv in over.items()) if over else "")


def _case(name, T, over, plant=False):
    c = synth.make_case(name, T=T, **over) if over or name == "tiny_fp32" else cached_case(name, T)
    c = synth.add_block_inputs(c)
    if plant:
        r = c.t["resid"]
        r[0] = 0                                      # zero row: normalises to zero
        if c.x_dtype == "bf16":
            r[1] = synth.bf16_bits(synth.bf16_to_f32(r[1]) * np.float32(2.0 ** 12))
        else:
            r[1] *= np.float32(2.0 ** 12)             # large row
    return c


def _sample(T, n, seed=3):
    if n is None or n >= T:
        return np.arange(T, dtype=np.int32)
    rng = np.random.default_rng(seed + T)
    s = set(rng.choice(T, n - 2, replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(s), np.int32)


def _f64(a, dt):
    return synth.bf16_to_f32(a).astype(np.float64) if dt == "bf16" else np.asarray(a, np.float64)


def _run(case, with_xn=True):
    cfg = config_of(case)
    w = device_weights(case)
    T, H = case.T, case.H
    tdt = torch.bfloat16 if case.x_dtype == "bf16" else torch.float32
    resid = to_torch(case.t["resid"])
    g = to_torch(case.t["norm_w"])
    out = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    xn = torch.empty((T, H), dtype=tdt, device="cuda") if with_xn else None
    lg = to_torch(case.t["logits"]) if case.drawn_logits else None
    idx = torch.empty((T, case.k), dtype=torch.int32, device="cuda")
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    moe.moe_forward_prenorm(cfg, w, g, case.norm_eps, resid, T, out, ws, xn=xn, logits=lg, topk_idx=idx)
    torch.cuda.synchronize()
    return cfg, w, out, xn, idx, ws


def _xn_bits(xn, dt):
    return xn.view(torch.int16).cpu().numpy().view(np.uint16) if dt == "bf16" else xn.cpu().numpy()


@pytest.mark.parametrize("p", BLOCKS, ids=_ids)
def test_prenorm_block_matches_oracle(p):
    name, T, nsample, over = p
    log("prenorm block %s" % _ids(p))
    case = _case(name, T, over, plant=(name == "tiny_fp32"))
    cfg, w, out, xn, idx, ws = _run(case)
    dt = case.x_dtype

    # 1. the normalised rows
    ref_xn = oracle.rmsnorm(case.t["resid"], case.t["norm_w"], case.norm_eps, dt)
    got_xn = _xn_bits(xn, dt)
    if dt == "bf16":
        diff = np.abs(got_xn.astype(np.int32) - ref_xn.astype(np.int32))
        assert diff.max() <= 1 and (diff == 0).mean() >= 0.999, "xn: %d elements differ, max %d bf16 steps" % (
            int((diff != 0).sum()), int(diff.max()))
    else:
        np.testing.assert_allclose(got_xn, ref_xn, rtol=2e-6, atol=1e-30)
    log("  xn: %d of %d elements off by one step" % (int((got_xn != ref_xn).sum()), got_xn.size))

    # 2. the residual add, exactly, against moe_forward on the GPU's own xn
    plain = torch.full_like(out, float("nan"))
    lg = to_torch(case.t["logits"]) if case.drawn_logits else None
    moe.moe_forward(cfg, w, xn, T, plain, ws, logits=lg)
    torch.cuda.synchronize()
    r32 = _f64(case.t["resid"], dt).astype(np.float32)
    assert np.array_equal(out.cpu().numpy(), r32 + plain.cpu().numpy())

    # 3. the layer part against the oracle's block
    tokens = _sample(T, nsample)
    rel = _check_block(case, tokens, idx, out, tol_of(case), "block layer part")
    log("  layer part: max|err|/max|ref| = %.3e (tol %.0e)" % (rel, tol_of(case)))


def test_prenorm_without_xn_output_is_identical():
    case = _case("qwen35moe_decode", 8, {})
    _, _, out_a, _, _, _ = _run(case, with_xn=True)
    _, _, out_b, _, _, _ = _run(case, with_xn=False)
    assert torch.equal(out_a, out_b)


def test_prenorm_zero_tokens_is_a_no_op():
    case = _case("qwen35moe_decode", 1, {})
    cfg = config_of(case)
    w = device_weights(case)
    out = torch.full((1, case.H), 7.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(moe.moe_workspace_bytes(cfg, 1), dtype=torch.uint8, device="cuda")
    moe.moe_forward_prenorm(cfg, w, to_torch(case.t["norm_w"]), 1e-6, to_torch(case.t["resid"]), 0, out, ws)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())

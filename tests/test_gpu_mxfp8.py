"""GPU MXFP8-activation mode (act_quant): the rounding kernel bit for bit
against the oracle's MXFP8 quantiser, and the MXFP4 layer with MXFP8 inputs
(few-token kernels on rounded bf16 values, the scaled MX MFMA grouped GEMM
for larger batches) against the oracle run in the same mode.

Tolerance: the MXFP4 one, max|err| <= 3e-2 * max|ref|.  Both sides round the
same inputs to the same MXFP8 values (x exactly; h from the GPU's bf16 h and
the oracle's double h, so a few h elements may land one E4M3 step apart)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_ffn_router_amd as moe
import synth
from tests._gpu import config_of, device_weights, h_numel, to_torch
from tests._parity import assert_normwise, check_layer_output, log

pytestmark = pytest.mark.gpu

TOL = 3e-2


def _bf16_rows(rng, rows, K):
    v = rng.standard_normal((rows, K)).astype(np.float32)
    v *= (2.0 ** rng.integers(-12, 12, size=(rows, 1))).astype(np.float32)
    v[0, :32] = 0.0                                   # all-zero block
    v[1, :32] *= 2.0 ** rng.integers(-20, 4, size=32)  # subnormal E4M3 elements
    v[2, 32:64] = 0.99 * np.sign(v[2, 32:64])        # saturating block (scaled max near 507)
    v[2, 40] = 1.0
    # exact ties between neighbouring E4M3 values (scale 2^-3)
    vals = np.array([oracle.e4m3_value(c) for c in range(0x09, 0x77)])
    mid = (vals[:-1] + vals[1:]) / 2
    v[3, :32] = (rng.choice(mid, 32) * 2.0 ** -3).astype(np.float32)
    v[3, 0] = 448.0 * 2.0 ** -3
    return synth.bf16_bits(v)


@pytest.mark.parametrize("rows,K", [(37, 320), (5, 64), (1, 2880), (300, 2048)])
def test_quantize_matches_oracle_bit_for_bit(rows, K):
    rng = np.random.default_rng(rows * 1000 + K)
    xb = _bf16_rows(rng, max(rows, 4), K)[:rows] if rows >= 4 else _bf16_rows(rng, 4, K)[:rows]
    stride = moe.mxfp8_scale_stride(K)
    codes = torch.empty((rows, K), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((rows, stride), dtype=torch.uint8, device="cuda")
    moe.moe_quantize_mxfp8(to_torch(xb), rows, K, codes, scales)
    torch.cuda.synchronize()
    ref_c, ref_s = oracle.mxfp8_quantize(synth.bf16_to_f32(xb).astype(np.float64))
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()[:, :K // 32]
    bad = np.nonzero(got_c != ref_c)
    assert bad[0].size == 0, "codes differ at %s: gpu %s oracle %s" % (
        list(zip(*bad))[:4], got_c[bad][:4], ref_c[bad][:4])
    assert np.array_equal(got_s, ref_s)


LAYERS = [
    ("gptoss20b_mxfp4", 16, None, dict(E=8, H=320, F=192, k=2)),     # few-token kernels, rounded bf16 inputs
    ("gptoss20b_mxfp4", 150, None, dict(E=8, H=320, F=192, k=2)),    # MX MFMA, a 64-deep last K step
    ("gptoss20b_mxfp4", 400, None, dict(E=4, H=256, F=128, k=2)),    # ~200-row segments, K multiple of 128
    ("gptoss20b_mxfp4", 97, None, dict(E=16, H=512, F=320, k=4)),    # ragged column tiles (F = 2.5 tiles)
    ("gptoss20b_mxfp4", 16, None, {}),                               # gpt-oss decode shape
    ("gptoss20b_mxfp4", 2048, 20, {}),                               # gpt-oss prefill shape, sampled tokens
    ("gptoss20b_mxfp4", 2000, 64, dict(E=8, H=384, F=2048, k=2)),   # 3 K steps, several tiles per workgroup
    ("gptoss20b_mxfp4", 300, 16, dict(E=4, H=4096, F=4096, k=2)),   # K = 4096: one tile per workgroup
]


def _ids(p):
    name, T, s, over = p
    return "%s-T%d%s" % (name, T, "-" + "-".join("%s%d" % kv for kv in over.items()) if over else "")


def _case(name, T, over):
    c = synth.make_case(name, T=T, **over)
    c.act_quant = "mxfp8"
    return c


def _sample(T, n, seed=1):
    if n is None or n >= T:
        return np.arange(T, dtype=np.int32)
    rng = np.random.default_rng(seed + T)
    s = set(rng.choice(T, n - 2, replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(s), np.int32)


@pytest.mark.parametrize("p", LAYERS, ids=_ids)
def test_forward_mxfp8_matches_oracle(p):
    name, T, nsample, over = p
    log("mxfp8 forward %s" % _ids(p))
    case = _case(name, T, over)
    cfg = config_of(case)
    w = device_weights(case)
    out = torch.full((T, case.H), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, case.k), dtype=torch.int32, device="cuda")
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    moe.moe_forward(cfg, w, to_torch(case.t["x"]), T, out, ws, topk_idx=idx)
    torch.cuda.synchronize()
    tokens = _sample(T, nsample)
    L = oracle.Layer(case)
    r_out, r_idx, _, _ = L.forward(tokens=tokens)
    rel = check_layer_output(case, tokens, idx.cpu().numpy(), out.cpu().numpy(), r_out, r_idx,
                             L.router_logits()[tokens], lambda gi, tk: L.forward(idx=gi, tokens=tk)[0], TOL,
                             "mxfp8 layer output")
    log("  max|err|/max|ref| = %.3e (tol %.0e)" % (rel, TOL))


@pytest.mark.parametrize("p", [LAYERS[i] for i in (0, 1, 3, 5)], ids=_ids)
def test_expert_ffn_and_combine_mxfp8(p):
    name, T, nsample, over = p
    log("mxfp8 expert_ffn/combine %s" % _ids(p))
    case = _case(name, T, over)
    cfg = config_of(case)
    w = device_weights(case)
    L = oracle.Layer(case)
    idx, wt = L.route(L.router_logits())
    off, sa, ap = oracle.permute(case.E, case.k, T, False, idx)
    nas = T * case.k
    d_off, d_sa = to_torch(off), to_torch(sa)
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    h = torch.empty(h_numel(case, T), dtype=torch.bfloat16, device="cuda")
    moe.moe_expert_ffn(cfg, w, to_torch(case.t["x"]), d_off, d_sa, T, h, ws)
    torch.cuda.synchronize()
    h_gpu = h.float().cpu().numpy().reshape(nas, case.F)
    xs = synth.bf16_to_f32(case.t["x"]).astype(np.float64)
    rows = np.arange(nas) if nsample is None else _sample(nas, 3 * nsample, seed=7)
    seg = np.searchsorted(off, rows, side="right") - 1
    ref = np.stack([L.expert_act(int(e), xs[sa[r] // case.k]) for r, e in zip(rows, seg)])
    rel = assert_normwise(h_gpu[rows], ref, TOL, "mxfp8 h")
    log("  h: max|err|/max|ref| = %.3e" % rel)

    # combine from the oracle's h rounded to bf16: both sides round the same
    # bf16 values to MXFP8
    tokens = np.arange(T) if nsample is None else _sample(T, nsample)
    h_in = np.zeros((nas, case.F), np.float32)
    for t in tokens:
        for j in range(case.k):
            p_ = int(ap[t * case.k + j])
            e = int(np.searchsorted(off, p_, side="right") - 1)
            h_in[p_] = synth.bf16_to_f32(synth.bf16_bits(L.expert_act(e, xs[t]).astype(np.float32)))
    out = torch.full((T, case.H), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_combine(cfg, w, to_torch(synth.bf16_bits(h_in.ravel())), d_off, d_sa, to_torch(wt), None, T, out, ws)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    refo = np.zeros((len(tokens), case.H))
    for i, t in enumerate(tokens):
        for j in range(case.k):
            p_ = int(ap[t * case.k + j])
            refo[i] += float(wt[t, j]) * L.expert_down(int(idx[t, j]), h_in[p_])
    rel = assert_normwise(out[tokens], refo, TOL, "mxfp8 combine output")
    log("  combine: max|err|/max|ref| = %.3e" % rel)


def test_mxfp8_step_needs_workspace():
    case = _case("gptoss20b_mxfp4", 16, dict(E=8, H=320, F=192, k=2))
    cfg = config_of(case)
    w = device_weights(case)
    off = torch.zeros(case.E + 1, dtype=torch.int32, device="cuda")
    sa = torch.zeros(16 * case.k, dtype=torch.int32, device="cuda")
    h = torch.empty(h_numel(case, 16), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_expert_ffn(cfg, w, to_torch(case.t["x"]), off, sa, 16, h)
    assert ei.value.status == moe.MOE_EWORKSPACE

"""GPU routing (moe_route) against the oracle: bit-exact expert indices on
the same logits, fp32 weights and shared gate within 1e-5 relative, planted
ties through the GPU router product, determinism."""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_ffn_router_amd as moe
import synth
from tests._gpu import config_of, device_weights, to_torch
from tests._parity import assert_rel, cached_case, log

pytestmark = pytest.mark.gpu

ROUTE_CASES = [("tiny_fp32", 8), ("qwen35moe_decode", 8), ("qwen35moe_prefill_zipf", 4096),
               ("gptoss20b_bf16", 2048), ("gptoss20b_mxfp4", 16), ("qwen35moe_decode", 333)]
ROUTE_ONLY = ("x", "router_w", "sh_gate_inp", "logits")


def _route(case, logits_np, with_router, ws=False):
    cfg = config_of(case)
    w = device_weights(case) if with_router else {k: v for k, v in device_weights(case).items()
                                                  if k not in ("router_w", "router_b")}
    T = case.T
    x = to_torch(case.t["x"]) if "x" in case.t else None
    lg = to_torch(np.ascontiguousarray(logits_np, np.float32)) if logits_np is not None else \
        torch.empty((T, case.E), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, case.k), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, case.k), dtype=torch.float32, device="cuda")
    sg = torch.empty(T, dtype=torch.float32, device="cuda") if case.has_shared else None
    scratch = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda") if ws else None
    moe.moe_route(cfg, w, x, lg, idx, wt, sg, T, scratch)
    torch.cuda.synchronize()
    return lg.cpu().numpy(), idx.cpu().numpy(), wt.cpu().numpy(), None if sg is None else sg.cpu().numpy()


@pytest.mark.parametrize("name,T", ROUTE_CASES)
def test_route_given_logits_matches_oracle(name, T):
    log("route given logits: %s T=%d" % (name, T))
    case = cached_case(name, T, ROUTE_ONLY) if name != "tiny_fp32" else synth.make_case(name, T=T)
    if case.drawn_logits:
        logits = case.t["logits"]
    else:
        logits = oracle_logits(case)
    _, idx, wt, sg = _route(case, logits, with_router=False)
    ref_idx, ref_w = route_ref(case, logits)
    assert np.array_equal(idx, ref_idx), "indices differ at tokens %s" % np.nonzero((idx != ref_idx).any(1))[0][:10]
    assert_rel(wt, ref_w, 1e-5, 1e-30, "routing weights")
    if case.has_shared:
        ref_s = oracle.sigmoid(shared_logit_ref(case))
        # the gate dot is fp32 on the GPU: allow its error bound through sigmoid' <= 1/4
        xs = np.abs(_f64(case.t["x"], case.x_dtype)) @ np.abs(_f64(case.t["sh_gate_inp"], case.x_dtype))
        bound = 0.25 * case.H * 2.0 ** -24 * xs
        assert np.all(np.abs(sg.astype(np.float64) - ref_s) <= 1e-5 * np.abs(ref_s) + bound)


def _f64(a, dt):
    return synth.bf16_to_f32(a).astype(np.float64) if dt == "bf16" else a.astype(np.float64)


def _layer_for_route(case):
    # the oracle's gating only needs the config; weights may be partial here
    return oracle.Layer(case)


def oracle_logits(case):
    return _layer_for_route(case).router_logits()


def shared_logit_ref(case):
    return _layer_for_route(case).shared_gate_logit()


def route_ref(case, logits):
    return _layer_for_route(case).route(logits)


def _hand_case(E, k, gating="softmax_topk", norm=True):
    c = synth.Case("hand", 1, 32, E, k, 32, 0, gating, norm, 1.0,
                   "swiglu" if gating == "softmax_topk" else "swiglu_oai", 1.702, 7.0, "f32", "f32", "f32")
    return c


HAND = [
    # (E, k, logits rows) with ties the first-seen rule must resolve
    (16, 3, [[0.5] * 16]),
    (16, 2, [[0, 1, 3, 0, 2, 3, 1, 0, 0, 0, 0, 0, 0, 0, 0, 0]]),
    (8, 2, [[-0.0, 0.0, -1, -1, -1, -1, -1, -1], [0.0, -0.0, -2, -3, -1, -1, -1, -1]]),
    (256, 8, None),   # built below: ties across lanes and register slots
    (1024, 32, None),
    (32, 4, [[1.0] * 32]),
]


@pytest.mark.parametrize("gating", ["softmax_topk", "topk_softmax"])
@pytest.mark.parametrize("hi", range(len(HAND)))
def test_route_hand_ties(hi, gating):
    E, k, rows = HAND[hi]
    if rows is None:
        rng = np.random.default_rng(E)
        lg = rng.integers(-3, 4, (64, E)).astype(np.float32) * np.float32(0.25)
        lg[0, [3, 67, 131, 195]] = 9.0   # same lane, different register slots
        lg[1, [5, 6, 7, 900 % E]] = 9.0   # neighbouring lanes
        lg[2, :] = -0.0
        lg[2, E - 1] = 0.0
    else:
        lg = np.array(rows, np.float32)
    case = _hand_case(E, k, gating)
    case.T = lg.shape[0]
    case.t["x"] = np.zeros((case.T, 32), np.float32)
    _, idx, wt, _ = _route(case, lg, with_router=False)
    ref_idx, ref_w = route_ref(case, lg)
    assert np.array_equal(idx, ref_idx)
    assert_rel(wt, ref_w, 1e-5, 1e-30, "weights")


@pytest.mark.parametrize("T", [8, 300])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_router_product_keeps_planted_ties(dtype, T):
    """Bit-equal router rows must give bit-equal GPU logits (every row is
    reduced in the same order, by the wave-per-row kernel for few tokens and
    by the MFMA kernel for many), so first-seen decides as on the CPU."""
    case = synth.make_case("tiny_fp32", T=T)
    if dtype == "bf16":
        case.x_dtype = case.w_dtype = case.router_dtype = "bf16"
        for n, a in list(case.t.items()):
            case.t[n] = synth.bf16_bits(a)
    lg, idx, wt, sg = _route(case, None, with_router=True)
    assert np.array_equal(lg[:, 4], lg[:, 9]) and np.array_equal(lg[:, 4], lg[:, 13])
    assert np.array_equal(lg[:, 7], lg[:, 12])
    assert list(idx[3]) == [4, 9] and list(idx[6]) == [0, 7]
    # GPU logits vs the oracle's, within the fp32 dot-product error bound
    L = oracle.Layer(case)
    ref = L.router_logits()
    xa = np.abs(_f64(case.t["x"], case.x_dtype))
    wa = np.abs(_f64(case.t["router_w"], case.router_dtype))
    bound = case.H * 2.0 ** -24 * (xa @ wa.T) + 2.0 ** -24 * np.abs(ref)
    assert np.all(np.abs(lg.astype(np.float64) - ref) <= bound)
    # and on identical logits the indices are the oracle's
    ref_idx, _ = L.route(lg)
    assert np.array_equal(idx, ref_idx)


@pytest.mark.parametrize("H,T", [(4096, 13), (4096, 64), (3072, 5), (2112, 9)])
def test_router_product_long_rows(H, T):
    """Router rows of 264 to 512 16-byte pieces (6 or 8 per lane, whole row in
    flight, 4 tokens per pass, a ragged last pass): bit-equal rows give
    bit-equal logits, the logits sit within the fp32 dot bound of the
    oracle's, the indices are the oracle's on them, and the shared gate
    (the extra row of the same kernel) is within 1e-5 relative plus the
    dot's fp32 bound through the sigmoid."""
    case = synth.make_case("qwen35moe_decode", T=T, E=64, H=H, F=64, Fs=64, k=4, only=set(ROUTE_ONLY))
    rw = case.t["router_w"]
    rw[41] = rw[3]
    rw[63] = rw[3]
    lg, idx, wt, sg = _route(case, None, with_router=True)
    assert np.array_equal(lg[:, 3], lg[:, 41]) and np.array_equal(lg[:, 3], lg[:, 63])
    L = oracle.Layer(case)
    ref = L.router_logits()
    xa = np.abs(_f64(case.t["x"], case.x_dtype))
    wa = np.abs(_f64(rw, case.router_dtype))
    bound = case.H * 2.0 ** -24 * (xa @ wa.T) + 2.0 ** -24 * np.abs(ref)
    assert np.all(np.abs(lg.astype(np.float64) - ref) <= bound)
    ref_idx, ref_w = L.route(lg)
    assert np.array_equal(idx, ref_idx)
    assert_rel(wt, ref_w, 1e-5, 1e-30, "routing weights")
    ref_s = oracle.sigmoid(shared_logit_ref(case))
    xs = np.abs(_f64(case.t["x"], case.x_dtype)) @ np.abs(_f64(case.t["sh_gate_inp"], case.x_dtype))
    assert np.all(np.abs(sg.astype(np.float64) - ref_s) <= 1e-5 * np.abs(ref_s) + 0.25 * case.H * 2.0 ** -24 * xs)


def test_router_product_split_over_hidden():
    """With scratch, a many-token bf16 router product runs in ranges of the
    hidden dimension summed by the gating kernel in a fixed order: logits
    within the fp32 bound of the oracle's, bit-equal router rows still give
    bit-equal logits, the indices are the oracle's on those logits, and two
    calls agree bit for bit."""
    case = synth.make_case("qwen35moe_decode", T=333, only=set(ROUTE_ONLY))
    rw = case.t["router_w"]
    rw[9] = rw[4]
    rw[13] = rw[4]
    rw[12] = rw[7]
    a = _route(case, None, with_router=True, ws=True)
    b = _route(case, None, with_router=True, ws=True)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    lg, idx = a[0], a[1]
    assert np.array_equal(lg[:, 4], lg[:, 9]) and np.array_equal(lg[:, 4], lg[:, 13])
    assert np.array_equal(lg[:, 7], lg[:, 12])
    L = oracle.Layer(case)
    ref = L.router_logits()
    xa = np.abs(_f64(case.t["x"], case.x_dtype))
    wa = np.abs(_f64(rw, case.router_dtype))
    bound = case.H * 2.0 ** -24 * (xa @ wa.T) + 2.0 ** -24 * np.abs(ref)
    assert np.all(np.abs(lg.astype(np.float64) - ref) <= bound)
    ref_idx, _ = L.route(lg)
    assert np.array_equal(idx, ref_idx)
    # the unsplit product (no scratch) is within the same bound
    c = _route(case, None, with_router=True)
    assert np.all(np.abs(c[0].astype(np.float64) - ref) <= bound)


def test_route_deterministic_and_T0():
    case = cached_case("qwen35moe_decode", 333, ROUTE_ONLY)
    a = _route(case, None, with_router=True)
    b = _route(case, None, with_router=True)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    cfg = config_of(case)
    moe.moe_route(cfg, device_weights(case), None, None, None, None, None, 0)  # T = 0: no-op


@pytest.mark.parametrize("E,k,T", [(256, 8, 8), (256, 8, 100), (32, 4, 64), (1024, 32, 20)])
def test_route_non_finite_logits_give_distinct_in_range_picks(E, k, T):
    """NaN and infinite logits are outside the contract, but the picks must
    still be k distinct experts in [0, E) for every token (the permutation
    and the expert kernels index by them).  Rows holding infinities but no
    NaN are ordered, so there the picks equal the oracle's."""
    log("route non-finite logits E=%d k=%d T=%d" % (E, k, T))
    rng = np.random.default_rng(E * 3 + T)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    nan_neg = np.array([0xFFFFFFFF], np.uint32).view(np.float32)[0]   # every bit set
    nan_pos = np.array([0x7FC00000], np.uint32).view(np.float32)[0]
    lg[0, :] = nan_neg                                  # a whole row of the all-ones NaN
    lg[1, : E // 2] = nan_neg
    lg[2, ::3] = nan_pos
    lg[3, :] = np.inf
    lg[4, 5] = np.inf
    lg[4, 9] = -np.inf
    lg[5, :] = -np.inf
    lg[6, rng.integers(0, E, 4)] = np.inf
    lg[7, ::2] = -np.inf
    for gating in ("softmax_topk", "topk_softmax"):
        c = synth.Case("nonfinite", T, 64, E, k, 64, 0, gating, True, 1.0, "swiglu", 1.702, 7.0,
                       "bf16", "bf16", "bf16")
        c.t["x"] = np.zeros((T, 64), np.uint16)
        _, idx, _, _ = _route(c, lg, with_router=False, ws=True)
        assert ((idx >= 0) & (idx < E)).all()
        assert all(len(set(r)) == k for r in idx.tolist()), "repeated pick"
        finite_order = ~np.isnan(lg).any(1)
        ref_idx, _ = route_ref(c, lg)
        assert np.array_equal(idx[finite_order], ref_idx[finite_order])

"""GPU permutation (moe_permute) against the oracle's stable counting sort:
offsets, sorted_assign and assign_pos bit-exact, on uniform, Zipf-skewed and
degenerate routings, across the one-workgroup / multi-workgroup boundary."""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_ffn_router_amd as moe
import synth
from tests._parity import log

pytestmark = pytest.mark.gpu


def _cfg(E, k, shared):
    return moe.MoeConfig(hidden=64, n_expert=E, top_k=k, expert_ff=64, shared_ff=64 if shared else 0,
                         x_dtype=moe.DTYPE_BF16, w_dtype=moe.DTYPE_BF16)


def _gpu_permute(E, k, T, shared, idx):
    cfg = _cfg(E, k, shared)
    n = T * k + (T if shared else 0)
    d_idx = torch.from_numpy(np.ascontiguousarray(idx, np.int32).reshape(-1)).cuda() if T else None
    off = torch.full((E + 1 + (1 if shared else 0),), -7, dtype=torch.int32, device="cuda")
    sa = torch.full((max(n, 1),), -7, dtype=torch.int32, device="cuda")
    ap = torch.full((max(n, 1),), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(moe.moe_workspace_bytes(cfg, T), 256), dtype=torch.uint8, device="cuda")
    moe.moe_permute(cfg, d_idx, T, off, sa, ap, ws)
    torch.cuda.synchronize()
    return off.cpu().numpy(), sa.cpu().numpy()[:n], ap.cpu().numpy()[:n]


def _uniform(E, k, T, seed):
    rng = np.random.default_rng(seed)
    return np.array([rng.permutation(E)[:k] for _ in range(T)], np.int32).reshape(T, k)


def _zipf(E, k, T):
    lg = synth.zipf_logits(T, E, 1.0)
    return np.argsort(-lg, axis=1, kind="stable")[:, :k].astype(np.int32)


CASES = [
    ("uniform", 16, 2, 8, True), ("uniform", 256, 8, 8, True), ("uniform", 32, 4, 16, False),
    ("uniform", 256, 8, 256, True),   # 2048 assignments: largest one-workgroup case
    ("uniform", 256, 8, 257, True),   # first multi-workgroup case, ragged last chunk
    ("zipf", 256, 8, 4096, True), ("uniform", 32, 4, 2048, False), ("uniform", 1024, 32, 100, False),
    ("uniform", 1024, 1, 3000, True), ("uniform", 4, 4, 700, False), ("uniform", 64, 3, 1, True),
    ("same", 256, 8, 1000, True), ("same", 16, 2, 5, False),
]


@pytest.mark.parametrize("kind,E,k,T,shared", CASES)
def test_permute_bit_exact(kind, E, k, T, shared):
    log("permute %s E=%d k=%d T=%d shared=%d" % (kind, E, k, T, shared))
    if kind == "uniform":
        idx = _uniform(E, k, T, E * 7 + T)
    elif kind == "zipf":
        idx = _zipf(E, k, T)
    else:  # every token picks the same experts: one long segment per pick
        idx = np.tile(np.arange(k, dtype=np.int32)[::-1], (T, 1))
    off, sa, ap = _gpu_permute(E, k, T, shared, idx)
    r_off, r_sa, r_ap = oracle.permute(E, k, T, shared, idx)
    assert np.array_equal(off, r_off)
    assert np.array_equal(sa, r_sa)
    assert np.array_equal(ap, r_ap)


def test_permute_T0_and_repeatable():
    off, sa, ap = _gpu_permute(16, 2, 0, True, np.zeros((0, 2), np.int32))
    assert np.all(off == -7)  # T = 0 is a no-op
    idx = _zipf(256, 8, 4096)
    a = _gpu_permute(256, 8, 4096, True, idx)
    b = _gpu_permute(256, 8, 4096, True, idx)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def _distinct_rule(idx, E):
    """The contract asks for k distinct picks in [0, E) per token; picks that
    break it (out of range, or repeating an earlier valid pick of the token)
    are replaced, in slot order, by the lowest experts the token's valid
    picks leave free.  Restated here from the header's description."""
    out = np.array(idx, np.int64)
    for t in range(out.shape[0]):
        valid, bad = [], []
        for j, e in enumerate(out[t]):
            if 0 <= e < E and e not in valid:
                valid.append(int(e))
            else:
                bad.append(j)
        free = (e for e in range(E) if e not in valid)
        for j in bad:
            out[t, j] = next(free)
    return out.astype(np.int32)


@pytest.mark.parametrize("E,k,T,shared", [(16, 4, 40, True), (64, 8, 300, False), (8, 8, 600, True)])
def test_permute_out_of_contract_picks_stay_a_bijection(E, k, T, shared):
    """Repeated, negative and too-large expert ids: every row is still placed
    exactly once (the expert kernels then never index past their buffers),
    by the documented replacement rule, in both kernel paths."""
    log("permute out-of-contract picks E=%d k=%d T=%d" % (E, k, T))
    rng = np.random.default_rng(E + k + T)
    idx = _uniform(E, k, T, T)
    idx[::3, 1] = idx[::3, 0]                          # a repeat of slot 0
    idx[1::5, k - 1] = E + rng.integers(0, 1000, idx[1::5].shape[0])
    idx[2::7, 0] = -1 - rng.integers(0, 5, idx[2::7].shape[0])
    idx[4] = idx[4, 0]                                 # one expert in every slot
    off, sa, ap = _gpu_permute(E, k, T, shared, idx)
    n = T * k + (T if shared else 0)
    assert np.array_equal(np.sort(sa), np.arange(n))   # a bijection
    assert np.array_equal(ap[sa], np.arange(n))
    fixed = _distinct_rule(idx, E)
    assert all(len(set(r)) == k for r in fixed.tolist())
    r_off, r_sa, r_ap = oracle.permute(E, k, T, shared, fixed)
    assert np.array_equal(off, r_off) and np.array_equal(sa, r_sa) and np.array_equal(ap, r_ap)

"""Pins of the oracle's token->expert permutation: brute-force stable sort,
bijection, histogram and segment offsets.  The pages only imply grouping
("grouped" launches, tokens sharing an expert streaming its weights once in
"qwen35moe - Forward-Pass Design", section "K80 GPU decode" and "Batched
prefill"); the order inside a segment is fixed here as ascending t*k + j."""
import numpy as np
import pytest

import oracle


def brute(E, k, T, shared, idx):
    n = T * k
    flat = np.asarray(idx).reshape(-1)
    keys = [(int(flat[a]), a) for a in range(n)] + ([(E, n + t) for t in range(T)] if shared else [])
    order = [a for _, a in sorted(keys)]
    return order


@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("E,k,T", [(16, 2, 8), (256, 8, 8), (32, 4, 37), (6, 6, 5), (4, 1, 1), (8, 3, 0)])
def test_permute_matches_brute_force(E, k, T, shared):
    rng = np.random.default_rng(E * 1000 + k * 10 + T)
    idx = np.array([rng.permutation(E)[:k] for _ in range(T)], np.int32).reshape(T, k)
    off, sa, ap = oracle.permute(E, k, T, shared, idx)
    n = T * k + (T if shared else 0)
    assert list(sa) == brute(E, k, T, shared, idx)
    # inverse permutation
    assert np.array_equal(sa[ap], np.arange(n)) and np.array_equal(ap[sa], np.arange(n))
    # offsets are the exclusive scan of the histogram
    cnt = np.bincount(idx.reshape(-1), minlength=E)
    if shared:
        cnt = np.append(cnt, T)
    assert off[0] == 0 and np.array_equal(np.diff(off), cnt) and off[-1] == n
    # every position lies in its expert's segment
    flat = idx.reshape(-1)
    for pos, a in enumerate(sa):
        e = flat[a] if a < T * k else E
        assert off[e] <= pos < off[e + 1]


def test_permute_skewed_and_empty_segments():
    E, k, T = 64, 4, 300
    rng = np.random.default_rng(1)
    # experts 0..3 take almost everything; most segments are empty
    idx = np.array([rng.permutation(6)[:k] for _ in range(T)], np.int32)
    off, sa, ap = oracle.permute(E, k, T, False, idx)
    assert list(sa) == brute(E, k, T, False, idx)
    assert np.all(np.diff(off)[6:] == 0)

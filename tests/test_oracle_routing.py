"""Pins of the oracle's gating (router logits, top-k, weights, shared gate)
against brute force, closed forms, invariants and hand-built ties.

Sources: "qwen35moe CPU-reference golden vectors", Kernel 4 (selection sort,
first-seen tie-break, pick order, renormalise then scale, sigmoid gate);
"Phase 19: MoE - gpt-oss-20b", section 2 Router (top-k then softmax over the
selected, router bias)."""
import itertools
import math

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle
import synth
from tests._cases import blank_case, small_random_case


def brute_topk(keys, k):
    # (key descending, index ascending): the order a first-seen selection sort yields
    return [e for e in sorted(range(len(keys)), key=lambda e: (-float(keys[e]), e))][:k]


@pytest.mark.parametrize("E,k", [(3, 1), (4, 2), (5, 3), (5, 5)])
def test_topk_exhaustive_small_integer_patterns(E, k):
    for pat in itertools.product([-1.0, 0.0, 1.0], repeat=E):
        keys = np.array(pat, np.float32)
        assert list(oracle.topk(keys, k)) == brute_topk(keys, k), pat


def test_topk_random_against_sort():
    rng = np.random.default_rng(7)
    for _ in range(300):
        E = int(rng.integers(1, 40))
        k = int(rng.integers(1, E + 1))
        keys = rng.integers(-3, 4, E).astype(np.float32) * np.float32(0.5)
        assert list(oracle.topk(keys, k)) == brute_topk(keys, k)


def test_topk_hand_ties():
    assert list(oracle.topk(np.zeros(8, np.float32), 3)) == [0, 1, 2]
    # a tie straddling the k boundary: experts 2 and 5 share the 2nd-best key
    assert list(oracle.topk(np.array([0, 1, 3, 0, 2, 3, 1], np.float32), 2)) == [2, 5]
    assert list(oracle.topk(np.array([0, 1, 3, 0, 2, 3, 1], np.float32), 3)) == [2, 5, 4]
    # -0 and +0 are equal keys: the first seen wins either way
    assert list(oracle.topk(np.array([-0.0, 0.0, -1.0], np.float32), 1)) == [0]
    assert list(oracle.topk(np.array([0.0, -0.0, -1.0], np.float32), 2)) == [0, 1]
    assert list(oracle.topk(np.array([-1.0, -0.0, 0.0], np.float32), 1)) == [1]


def test_topk_invariants():
    rng = np.random.default_rng(11)
    for _ in range(100):
        E, k = 64, 8
        keys = rng.standard_normal(E).astype(np.float32)
        idx = oracle.topk(keys, k)
        # scaling by 2 is exact in fp32 and order preserving
        assert list(oracle.topk(keys * np.float32(2), k)) == list(idx)
        # relabelling experts relabels the picks (no ties in continuous draws)
        perm = rng.permutation(E)
        relabelled = np.empty_like(keys)
        relabelled[perm] = keys
        assert list(oracle.topk(relabelled, k)) == [int(perm[i]) for i in idx]


def _route_case(E, k, gating="softmax_topk", norm=True, scale=1.0):
    return oracle.Layer(blank_case(1, 32, E, k, 16, gating=gating, norm=norm, scale=scale))


def test_weights_sum_to_scale_and_k1():
    rng = np.random.default_rng(3)
    for scale in (1.0, 2.5):
        L = _route_case(64, 8, scale=scale)
        lg = rng.standard_normal((50, 64)).astype(np.float32) * 3
        idx, w = L.route(lg)
        assert np.all(np.abs(w.astype(np.float64).sum(1) - scale) <= 8 * np.spacing(np.float32(scale)))
        L1 = _route_case(64, 1, scale=scale)
        _, w1 = L1.route(lg)
        assert np.all(w1 == np.float32(scale))


def test_weights_k2_closed_form_and_equal_logits():
    for gating in ("softmax_topk", "topk_softmax"):
        L = _route_case(16, 2, gating=gating)
        rng = np.random.default_rng(5)
        lg = rng.standard_normal((40, 16)).astype(np.float32)
        idx, w = L.route(lg)
        for t in range(40):
            l0, l1 = float(lg[t, idx[t, 0]]), float(lg[t, idx[t, 1]])
            assert abs(float(w[t, 0]) - 1.0 / (1.0 + math.exp(l1 - l0))) <= 2e-7
        Lk = _route_case(16, 4, gating=gating)
        idx, w = Lk.route(np.full((1, 16), 0.75, np.float32))
        assert list(idx[0]) == [0, 1, 2, 3] and np.all(w == np.float32(0.25))


def test_softmax_without_renorm_matches_library_softmax():
    L = _route_case(32, 4, norm=False)
    rng = np.random.default_rng(9)
    lg = rng.standard_normal((20, 32)).astype(np.float32) * 4
    idx, w = L.route(lg)
    p = softmax(lg.astype(np.float64), axis=1)
    for t in range(20):
        ref = p[t, idx[t]]
        assert np.allclose(w[t], ref, rtol=1e-6, atol=0)


def test_qwen_renorm_equals_gptoss_topk_softmax():
    """softmax -> top-k -> renormalise == top-k -> softmax (zero bias): the full
    softmax denominator cancels."""
    rng = np.random.default_rng(13)
    lg = rng.standard_normal((64, 64)).astype(np.float32) * 2
    iq, wq = _route_case(64, 8, "softmax_topk").route(lg)
    ig, wg = _route_case(64, 8, "topk_softmax").route(lg)
    assert np.array_equal(iq, ig)
    assert np.all(np.abs(wq - wg) <= 4 * np.spacing(np.maximum(np.abs(wq), np.abs(wg))))


def test_prob_key_reading_agrees_on_seeded_logits():
    L = _route_case(256, 8)
    assert L.prob_key_disagreements(synth.zipf_logits(1024, 256)) == 0


def test_router_logits_exact_integer_case_and_bias():
    """Small integers: every product and sum is exact, so the logits equal the
    integer matrix product (a transposed operand or wrong index would not)."""
    rng = np.random.default_rng(17)
    c = blank_case(3, 32, 8, 2, 16, gating="topk_softmax", act="swiglu_oai")
    c.t["x"] = rng.integers(-4, 5, (3, 32)).astype(np.float32)
    c.t["router_w"] = rng.integers(-4, 5, (8, 32)).astype(np.float32)
    c.t["router_b"] = rng.integers(-4, 5, 8).astype(np.float32)
    lg = oracle.Layer(c).router_logits()
    ref = c.t["x"].astype(np.int64) @ c.t["router_w"].astype(np.int64).T + c.t["router_b"].astype(np.int64)
    assert np.array_equal(lg, ref.astype(np.float32))


def test_shared_gate_exact_integer_case():
    """Small integers make the shared-gate dot exact: sh_gate_inp . x equals
    the int64 product, in the step function and inside the whole layer (whose
    gate is sigmoid of that dot).  The router rows and the shared expert's own
    matrices hold other integers, so reading the wrong tensor, or the wrong
    row of x, fails."""
    rng = np.random.default_rng(29)
    T, H = 5, 64
    c = blank_case(T, H, 8, 2, 32, Fs=32)
    c.t["x"] = rng.integers(-3, 4, (T, H)).astype(np.float32)
    c.t["sh_gate_inp"] = rng.integers(-3, 4, H).astype(np.float32)
    c.t["router_w"] = rng.integers(-3, 4, (8, H)).astype(np.float32)
    c.t["sh_gate_w"] = rng.integers(-3, 4, (32, H)).astype(np.float32)
    c.t["sh_up_w"] = rng.integers(-3, 4, (32, H)).astype(np.float32)
    ref = c.t["x"].astype(np.int64) @ c.t["sh_gate_inp"].astype(np.int64)
    assert len(set(ref.tolist())) > 2          # the tokens' gates differ
    L = oracle.Layer(c)
    assert np.array_equal(L.shared_gate_logit(), ref.astype(np.float32))
    _, _, _, sg = L.forward()
    want = expit(ref.astype(np.float64)).astype(np.float32)
    assert np.all(np.abs(sg - want) <= np.spacing(want))


def test_shared_gate_closed_forms():
    assert oracle.sigmoid(np.array([0.0], np.float32))[0] == np.float32(0.5)
    assert abs(float(oracle.sigmoid(np.array([math.log(3.0)], np.float32))[0]) - 0.75) < 1e-7
    s = np.linspace(-20, 20, 101).astype(np.float32)
    assert np.allclose(oracle.sigmoid(s), expit(s.astype(np.float64)), rtol=1e-7, atol=1e-30)
    # x = 0 gives a zero gate dot and a gate of exactly 0.5
    c = small_random_case()
    c.t["x"] = np.zeros_like(c.t["x"])
    _, _, _, sg = oracle.Layer(c).forward()
    assert np.all(sg == np.float32(0.5))


def test_tiny_case_planted_ties():
    """The tiny layer plants bit-equal router rows (9 = 13 = 4, 12 = 7): token 3
    ties experts 4, 9, 13 at the top and first-seen keeps 4 then 9; token 6 has
    expert 0 first and 7, 12 tied for second, so 7 is kept."""
    c = synth.make_case("tiny_fp32")
    L = oracle.Layer(c)
    lg = L.router_logits()
    assert lg[3, 4] == lg[3, 9] == lg[3, 13]
    assert lg[6, 7] == lg[6, 12]
    idx, w = L.route(lg)
    assert list(idx[3]) == [4, 9]
    assert list(idx[6]) == [0, 7]
    assert w[3, 0] == w[3, 1] == np.float32(0.5)

"""Pins of the oracle's expert FFNs, combine and whole layer.

Sources: "qwen35moe - Forward-Pass Design", section "Shared-expert MoE FFN"
(SwiGLU experts, sigmoid-gated shared expert, out = moe_out + sgate*shexp);
"Phase 19: MoE - gpt-oss-20b", section 2 Experts (interleaved gate_up with
bias, gate clamped above, up clamped both ways, (up+1)*gate*sigmoid(1.702
gate), down + bias inside the weighted sum) and Router (dense scatter form).
Structured weights (one-hot rows) make each result a closed form, so a
transposed operand, a swapped gate/up or a dropped term fails."""
import math

import numpy as np
import pytest

import oracle
import synth
from tests._cases import blank_case, small_random_case


def sig(v):
    return 1.0 / (1.0 + math.exp(-v))


def test_swiglu_one_hot_closed_form():
    # gate row f reads x[2f], up row f reads x[2f+1]; down row o reads h[o % F]
    T, H, E, k, F = 2, 16, 2, 1, 8
    c = blank_case(T, H, E, k, F)
    c.t["x"] = (np.arange(T * H, dtype=np.float32).reshape(T, H) - 9.0) * np.float32(0.25)
    for f in range(F):
        c.t["gate_w"][1, f, 2 * f] = 1.0
        c.t["up_w"][1, f, 2 * f + 1] = 1.0
    for o in range(H):
        c.t["down_w"][1, o, o % F] = 2.0
    c.t["router_w"][1, :] = 1.0  # every token picks expert 1 (x sums positive/negative: use bias-free tie check below)
    L = oracle.Layer(c)
    for t in range(T):
        h = L.expert_act(1, c.t["x"][t].astype(np.float64))
        for f in range(F):
            g, u = float(c.t["x"][t, 2 * f]), float(c.t["x"][t, 2 * f + 1])
            assert abs(h[f] - g * sig(g) * u) <= 1e-15 * max(1.0, abs(h[f]))
        y = L.expert_down(1, h)
        assert np.allclose(y, [2.0 * h[o % F] for o in range(H)], rtol=0, atol=1e-14)
        # expert 0 has zero weights: its activation vanishes
        assert np.all(L.expert_act(0, c.t["x"][t].astype(np.float64)) == 0.0)


def test_oai_interleave_clamp_closed_form():
    """Even gate_up rows are the gate, odd rows the up projection.  Row 2f reads
    x[f], row 2f+1 reads x[F+f]; biases shift them.  Includes clamp hits."""
    T, H, E, k, F = 1, 32, 1, 1, 16
    c = blank_case(T, H, E, k, F, gating="topk_softmax", act="swiglu_oai")
    x = np.array([10.0, -10.0, 3.0, -2.0, 0.5, 7.5, -7.5, 0.0] * 4, np.float32)
    x[F] = -10.0  # up input of f = 0, whose gate input is 10
    c.t["x"][0] = x
    for f in range(F):
        c.t["gate_up_w"][0, 2 * f, f] = 1.0
        c.t["gate_up_w"][0, 2 * f + 1, F + f] = 1.0
    c.t["gate_up_b"][0, 2 * 3] = 0.25     # gate bias of f=3
    c.t["gate_up_b"][0, 2 * 5 + 1] = -0.5  # up bias of f=5
    h = oracle.Layer(c).expert_act(0, x.astype(np.float64))
    for f in range(F):
        g = float(x[f]) + (0.25 if f == 3 else 0.0)
        u = float(x[F + f]) + (-0.5 if f == 5 else 0.0)
        g = min(g, 7.0)
        u = max(-7.0, min(7.0, u))
        a = float(np.float32(1.702))
        ref = (u + 1.0) * g * sig(a * g)
        assert abs(h[f] - ref) <= 1e-14 * max(1.0, abs(ref)), f
    # the named clamp case: gate 10 -> 7, up -10 -> -7 => (-7 + 1) * 7 * sigmoid(1.702 * 7)
    assert abs(h[0] - (-6.0 * 7.0 * sig(float(np.float32(1.702)) * 7.0))) < 1e-12


def test_oai_zero_input_gives_bias_closed_form():
    c = small_random_case(act="swiglu_oai", gating="topk_softmax", Fs=0)
    c.t["x"] = np.zeros_like(c.t["x"])
    L = oracle.Layer(c)
    out, idx, w, _ = L.forward()
    a = float(np.float32(1.702))
    for t in range(c.T):
        ref = np.zeros(c.H)
        for j in range(c.k):
            e = idx[t, j]
            bg = c.t["gate_up_b"][e, 0::2].astype(np.float64)
            bu = c.t["gate_up_b"][e, 1::2].astype(np.float64)
            g = np.minimum(bg, 7.0)
            u = np.clip(bu, -7.0, 7.0)
            h0 = (u + 1.0) * g / (1.0 + np.exp(-a * g))
            y = c.t["down_w"][e].astype(np.float64) @ h0 + c.t["down_b"][e]
            ref += float(w[t, j]) * y
        assert np.allclose(out[t], ref, rtol=1e-6, atol=1e-6)


def test_qwen_zero_input_gives_zero():
    c = small_random_case()
    c.t["x"] = np.zeros_like(c.t["x"])
    out, _, _, sg = oracle.Layer(c).forward()
    assert np.all(out == 0.0) and np.all(sg == np.float32(0.5))


@pytest.mark.parametrize("act,gating,Fs", [("swiglu", "softmax_topk", 32), ("swiglu", "softmax_topk", 0),
                                           ("swiglu_oai", "topk_softmax", 0)])
def test_sparse_equals_dense_brute_force(act, gating, Fs):
    c = small_random_case(T=7, act=act, gating=gating, Fs=Fs)
    L = oracle.Layer(c)
    out, _, _, _ = L.forward()
    dense = L.forward_dense()
    assert np.all(np.abs(out - dense) <= 1e-6 * np.abs(dense).max())
    # and the permuted path (expert_ffn -> combine) agrees with the token path
    lg = L.router_logits()
    idx, w = L.route(lg)
    sg = oracle.sigmoid(L.shared_gate_logit()) if Fs else None
    off, sa, _ = oracle.permute(c.E, c.k, c.T, Fs > 0, idx)
    h = L.expert_ffn(off, sa)
    out2 = L.combine(h, off, sa, w, sg)
    assert np.all(np.abs(out2 - dense) <= 1e-5 * np.abs(dense).max())


@pytest.mark.parametrize("F,Fs", [(32, 64), (64, 32)])
def test_permuted_path_with_shared_width_unlike_routed(F, Fs):
    """h holds the T*k routed rows of F values, then the T shared rows of Fs
    values; with F != Fs the permuted path (expert_ffn -> combine) must still
    equal the dense brute force."""
    c = small_random_case(T=6, F=F, Fs=Fs)
    L = oracle.Layer(c)
    dense = L.forward_dense()
    idx, w = L.route(L.router_logits())
    sg = oracle.sigmoid(L.shared_gate_logit())
    off, sa, _ = oracle.permute(c.E, c.k, c.T, True, idx)
    h = L.expert_ffn(off, sa)
    assert h.size == c.T * c.k * F + c.T * Fs
    out = L.combine(h, off, sa, w, sg)
    assert np.all(np.abs(out - dense) <= 1e-5 * np.abs(dense).max())


def test_identical_experts_reduce_to_one_ffn():
    """All routed experts equal => sum of weights (= 1) times that FFN."""
    c = small_random_case(T=4, Fs=0)
    for n in ("gate_w", "up_w", "down_w"):
        c.t[n][:] = c.t[n][0]
    L = oracle.Layer(c)
    out, _, _, _ = L.forward()
    for t in range(c.T):
        y = L.expert_down(0, L.expert_act(0, c.t["x"][t].astype(np.float64)))
        assert np.allclose(out[t], y, rtol=1e-6, atol=1e-7)


def test_single_expert_isolation_k1():
    """k = 1 with renormalisation gives weight exactly 1: out = FFN_e(x) + sgate*shared."""
    c = small_random_case(T=4, k=1)
    L = oracle.Layer(c)
    out, idx, w, sg = L.forward()
    assert np.all(w == 1.0)
    for t in range(c.T):
        xr = c.t["x"][t].astype(np.float64)
        y = L.expert_down(idx[t, 0], L.expert_act(idx[t, 0], xr))
        ys = L.expert_down(c.E, L.expert_act(c.E, xr))
        assert np.allclose(out[t], y + float(sg[t]) * ys, rtol=1e-6, atol=1e-7)


def test_fp32_layer_error_bound_vs_float64():
    """The tiny fp32 layer computed in fp32 stays within the fp32 dot-product
    error bound of the double-accumulating oracle (Higham, Accuracy and
    Stability of Numerical Algorithms, 2nd ed., section 3.1: |err| <= n u sum|a b|)."""
    c = synth.make_case("tiny_fp32")
    L = oracle.Layer(c)
    lg = L.router_logits()
    x = c.t["x"].astype(np.float32)
    lg32 = np.zeros_like(lg)
    for t in range(c.T):
        for e in range(c.E):
            acc = np.float32(0)
            for hh in range(c.H):
                acc = np.float32(acc + x[t, hh] * c.t["router_w"][e, hh])
            lg32[t, e] = acc
    bound = c.H * 2.0 ** -24 * (np.abs(x.astype(np.float64)) @ np.abs(c.t["router_w"].astype(np.float64)).T)
    assert np.all(np.abs(lg32.astype(np.float64) - lg) <= bound + 2.0 ** -24 * np.abs(lg))

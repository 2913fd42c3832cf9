"""Hand-built small layers for pinning the oracle (structured weights whose
results have closed forms)."""
import numpy as np

import synth


def blank_case(T, H, E, k, F, Fs=0, gating="softmax_topk", norm=True, scale=1.0, act="swiglu",
               w_dtype="f32", x_dtype="f32", router_dtype="f32"):
    c = synth.Case("hand", T, H, E, k, F, Fs, gating, norm, scale, act, 1.702, 7.0,
                   x_dtype, w_dtype, router_dtype)
    c.t["x"] = np.zeros((T, H), np.float32)
    c.t["router_w"] = np.zeros((E, H), np.float32)
    if act == "swiglu":
        c.t["gate_w"] = np.zeros((E, F, H), np.float32)
        c.t["up_w"] = np.zeros((E, F, H), np.float32)
    else:
        c.t["gate_up_w"] = np.zeros((E, 2 * F, H), np.float32)
        c.t["gate_up_b"] = np.zeros((E, 2 * F), np.float32)
        c.t["down_b"] = np.zeros((E, H), np.float32)
    c.t["down_w"] = np.zeros((E, H, F), np.float32)
    if Fs:
        c.t["sh_gate_w"] = np.zeros((Fs, H), np.float32)
        c.t["sh_up_w"] = np.zeros((Fs, H), np.float32)
        c.t["sh_down_w"] = np.zeros((H, Fs), np.float32)
        c.t["sh_gate_inp"] = np.zeros(H, np.float32)
    return c


def small_random_case(T=5, H=64, E=6, k=2, F=32, Fs=32, act="swiglu", gating="softmax_topk",
                      seed=0x1234567, norm=True):
    """fp32 random layer small enough for dense brute force."""
    c = synth.Case("small", T, H, E, k, F, Fs, gating, norm, 1.0, act, 1.702, 7.0, "f32", "f32", "f32")
    c.t["x"] = synth.normal("x", (T, H), 1.0, "f32", seed)
    c.t["router_w"] = synth.normal("router_w", (E, H), 1.0 / np.sqrt(H), "f32", seed)
    if act == "swiglu":
        c.t["gate_w"] = synth.normal("gate_w", (E, F, H), 1.0 / np.sqrt(H), "f32", seed)
        c.t["up_w"] = synth.normal("up_w", (E, F, H), 1.0 / np.sqrt(H), "f32", seed)
    else:
        c.t["router_b"] = synth.normal("router_b", (1, E), 1.0 / np.sqrt(H), "f32", seed)[0]
        c.t["gate_up_w"] = synth.normal("gate_up_w", (E, 2 * F, H), 3.0 / np.sqrt(H), "f32", seed)
        c.t["gate_up_b"] = synth.normal("gate_up_b", (E, 2 * F), 1.0, "f32", seed)
        c.t["down_b"] = synth.normal("down_b", (E, H), 1.0 / np.sqrt(F), "f32", seed)
    c.t["down_w"] = synth.normal("down_w", (E, H, F), 1.0 / np.sqrt(F), "f32", seed)
    if Fs:
        c.t["sh_gate_w"] = synth.normal("sh_gate_w", (Fs, H), 1.0 / np.sqrt(H), "f32", seed)
        c.t["sh_up_w"] = synth.normal("sh_up_w", (Fs, H), 1.0 / np.sqrt(H), "f32", seed)
        c.t["sh_down_w"] = synth.normal("sh_down_w", (H, Fs), 1.0 / np.sqrt(Fs), "f32", seed)
        c.t["sh_gate_inp"] = synth.normal("sh_gate_inp", (1, H), 1.0 / np.sqrt(H), "f32", seed)[0]
    return c

"""Test/bench plumbing: upload a synthetic layer case to the GPU and build
the binding's config for it."""
import numpy as np
import torch

import sparse_moe_ffn_router_amd as moe

_DT = {"f32": moe.DTYPE_F32, "bf16": moe.DTYPE_BF16, "mxfp4": moe.DTYPE_MXFP4}


def config_of(case) -> "moe.MoeConfig":
    return moe.MoeConfig(
        hidden=case.H, n_expert=case.E, top_k=case.k, expert_ff=case.F, shared_ff=case.Fs,
        gating=moe.GATING_SOFTMAX_TOPK if case.gating == "softmax_topk" else moe.GATING_TOPK_SOFTMAX,
        norm_topk_prob=case.norm_topk_prob, weights_scale=case.weights_scale,
        act=moe.ACT_SWIGLU if case.act == "swiglu" else moe.ACT_SWIGLU_OAI,
        act_alpha=case.alpha, act_limit=case.limit, x_dtype=_DT[case.x_dtype], w_dtype=_DT[case.w_dtype],
        act_quant=moe.ACT_QUANT_MXFP8 if case.act_quant == "mxfp8" else moe.ACT_QUANT_NONE)


def to_torch(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def x_tensor(case, x: np.ndarray, device="cuda"):
    return to_torch(x, device)


def device_weights(case, device="cuda", router=True):
    """dict of device tensors named as moe_weights fields."""
    t = case.t
    w = {}
    if router and "router_w" in t and not case.drawn_logits:
        w["router_w"] = to_torch(t["router_w"], device)
        if "router_b" in t:
            w["router_b"] = to_torch(t["router_b"], device)
    names = {"gate_w": "gate_w", "up_w": "up_w", "gate_up_w": "gate_up_w", "gate_up_b": "gate_up_b",
             "down_w": "down_w", "down_b": "down_b", "sh_gate_w": "sh_gate_w", "sh_up_w": "sh_up_w",
             "sh_down_w": "sh_down_w", "sh_gate_inp": "sh_gate_inp"}
    for k, n in names.items():
        if k in t:
            w[n] = to_torch(t[k], device)
    if case.w_dtype == "mxfp4":
        for field, key in (("gate_up_w", "gate_up_codes"), ("gate_up_scales", "gate_up_scales"),
                           ("down_w", "down_codes"), ("down_scales", "down_scales")):
            if key in t:
                w[field] = to_torch(t[key], device)
    return w


def h_numel(case, T):
    return T * case.k * case.F + (T * case.Fs if case.has_shared else 0)


def act_dtype(case):
    return torch.float32 if case.x_dtype == "f32" else torch.bfloat16

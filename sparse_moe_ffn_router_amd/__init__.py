"""Python binding of libmoe (include/moe.h): the MI355X sparse MoE FFN layer.

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libmoe.so``.  Tensors are torch device tensors (PyTorch supplies device
memory and streams); the functions mirror the C entry points one to one and
raise ``MoeError`` on a non-zero status.  There is no CPU fallback: importing
this package fails if ``libmoe.so`` has not been built
(``python sparse_moe_ffn_router_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = 0, -1, -2, -3, -4
DTYPE_F32, DTYPE_BF16, DTYPE_MXFP4 = 0, 1, 2
GATING_SOFTMAX_TOPK, GATING_TOPK_SOFTMAX = 0, 1
ACT_SWIGLU, ACT_SWIGLU_OAI = 0, 1
ACT_QUANT_NONE, ACT_QUANT_MXFP8 = 0, 1

EXPORTS = ("moe_workspace_bytes", "moe_route", "moe_permute", "moe_expert_ffn", "moe_combine",
           "moe_forward", "moe_forward_noalloc", "moe_forward_prenorm", "moe_quantize_mxfp8",
           "moe_status_string")
NOALLOC_SCRATCH_BYTES = 32 << 20  # MOE_NOALLOC_SCRATCH_BYTES


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s failed: %s (status %d)" % (what, status_string(status), status))
        self.status = status


class _Config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_expert", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("expert_ff", ctypes.c_int32), ("shared_ff", ctypes.c_int32), ("gating", ctypes.c_int32),
                ("norm_topk_prob", ctypes.c_int32), ("weights_scale", ctypes.c_float),
                ("act", ctypes.c_int32), ("act_alpha", ctypes.c_float), ("act_limit", ctypes.c_float),
                ("x_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32), ("act_quant", ctypes.c_int32)]


_WEIGHT_FIELDS = ("router_w", "router_b", "gate_w", "up_w", "gate_up_w", "gate_up_scales", "gate_up_b",
                  "down_w", "down_scales", "down_b", "sh_gate_w", "sh_up_w", "sh_down_w", "sh_gate_inp")


class _Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _WEIGHT_FIELDS]


@dataclass
class MoeConfig:
    hidden: int
    n_expert: int
    top_k: int
    expert_ff: int
    shared_ff: int = 0
    gating: int = GATING_SOFTMAX_TOPK
    norm_topk_prob: bool = True
    weights_scale: float = 1.0
    act: int = ACT_SWIGLU
    act_alpha: float = 1.702
    act_limit: float = 7.0
    x_dtype: int = DTYPE_BF16
    w_dtype: int = DTYPE_BF16
    act_quant: int = ACT_QUANT_NONE

    def _c(self) -> _Config:
        return _Config(self.hidden, self.n_expert, self.top_k, self.expert_ff, self.shared_ff, self.gating,
                       int(self.norm_topk_prob), self.weights_scale, self.act, self.act_alpha, self.act_limit,
                       self.x_dtype, self.w_dtype, self.act_quant)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libmoe.so is not built (%s); run python sparse_moe_ffn_router_amd/build.py" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    C, W = ctypes.POINTER(_Config), ctypes.POINTER(_Weights)
    L.moe_workspace_bytes.argtypes = [C, i32]
    L.moe_workspace_bytes.restype = sz
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_route.argtypes = [C, W, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    L.moe_permute.argtypes = [C, vp, i32, vp, vp, vp, vp, sz, vp]
    L.moe_expert_ffn.argtypes = [C, W, vp, vp, vp, i32, vp, vp, sz, vp]
    L.moe_combine.argtypes = [C, W, vp, vp, vp, vp, vp, i32, vp, vp, sz, vp]
    L.moe_forward.argtypes = [C, W, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_forward_noalloc.argtypes = [C, W, vp, i32, vp, vp, vp, vp, vp, vp]
    L.moe_forward_prenorm.argtypes = [C, W, vp, ctypes.c_float, vp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_quantize_mxfp8.argtypes = [vp, ctypes.c_int64, i32, vp, vp, vp]
    return L


lib = _load()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _weights(w) -> _Weights:
    """w: mapping (or object with attributes) of device tensors named as in moe_weights."""
    get = (lambda n: w.get(n)) if isinstance(w, dict) else (lambda n: getattr(w, n, None))
    return _Weights(*[_ptr(get(n)) for n in _WEIGHT_FIELDS])


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoeError(status, what)


def status_string(status: int) -> str:
    return lib.moe_status_string(status).decode()


def moe_status_string(status: int) -> str:
    return status_string(status)


def moe_workspace_bytes(cfg: MoeConfig, T: int) -> int:
    return int(lib.moe_workspace_bytes(ctypes.byref(cfg._c()), T))


def moe_route(cfg, w, x, logits, topk_idx, topk_w, sgate, T, ws=None, stream=None, ws_bytes=None):
    c, ww = cfg._c(), _weights(w)
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(lib.moe_route(ctypes.byref(c), ctypes.byref(ww), _ptr(x), _ptr(logits), _ptr(topk_idx), _ptr(topk_w),
                         _ptr(sgate), T, _ptr(ws), nb, _stream(stream)), "moe_route")


def moe_permute(cfg, topk_idx, T, offsets, sorted_assign, assign_pos, ws, stream=None, ws_bytes=None):
    c = cfg._c()
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(lib.moe_permute(ctypes.byref(c), _ptr(topk_idx), T, _ptr(offsets), _ptr(sorted_assign),
                           _ptr(assign_pos), _ptr(ws), nb, _stream(stream)), "moe_permute")


def moe_expert_ffn(cfg, w, x, offsets, sorted_assign, T, h, ws=None, stream=None, ws_bytes=None):
    c, ww = cfg._c(), _weights(w)
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(lib.moe_expert_ffn(ctypes.byref(c), ctypes.byref(ww), _ptr(x), _ptr(offsets), _ptr(sorted_assign), T,
                              _ptr(h), _ptr(ws), nb, _stream(stream)), "moe_expert_ffn")


def moe_combine(cfg, w, h, offsets, sorted_assign, topk_w, sgate, T, out, ws, stream=None, ws_bytes=None):
    c, ww = cfg._c(), _weights(w)
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(lib.moe_combine(ctypes.byref(c), ctypes.byref(ww), _ptr(h), _ptr(offsets), _ptr(sorted_assign),
                           _ptr(topk_w), _ptr(sgate), T, _ptr(out), _ptr(ws), nb, _stream(stream)), "moe_combine")


def moe_forward(cfg, w, x, T, out, ws, logits=None, topk_idx=None, topk_w=None, sgate=None, stream=None,
                ws_bytes=None):
    c, ww = cfg._c(), _weights(w)
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(lib.moe_forward(ctypes.byref(c), ctypes.byref(ww), _ptr(x), T, _ptr(out), _ptr(logits), _ptr(topk_idx),
                           _ptr(topk_w), _ptr(sgate), _ptr(ws), nb, _stream(stream)), "moe_forward")


def moe_forward_noalloc(cfg, w, x, T, out, logits=None, topk_idx=None, topk_w=None, sgate=None, stream=None):
    """moe_forward with the library's built-in scratch (no workspace argument,
    nothing allocated)."""
    c, ww = cfg._c(), _weights(w)
    _check(lib.moe_forward_noalloc(ctypes.byref(c), ctypes.byref(ww), _ptr(x), T, _ptr(out), _ptr(logits),
                                   _ptr(topk_idx), _ptr(topk_w), _ptr(sgate), _stream(stream)),
           "moe_forward_noalloc")


def moe_forward_prenorm(cfg, w, norm_w, norm_eps, resid, T, out, ws, xn=None, logits=None, topk_idx=None,
                        topk_w=None, sgate=None, stream=None, ws_bytes=None):
    """out = resid + layer(RMSNorm(resid) * norm_w); xn optionally receives
    the normalised rows."""
    c, ww = cfg._c(), _weights(w)
    nb = _nbytes(ws) if ws_bytes is None else ws_bytes
    _check(lib.moe_forward_prenorm(ctypes.byref(c), ctypes.byref(ww), _ptr(norm_w), float(norm_eps), _ptr(resid),
                                   T, _ptr(out), _ptr(xn), _ptr(logits), _ptr(topk_idx), _ptr(topk_w),
                                   _ptr(sgate), _ptr(ws), nb, _stream(stream)), "moe_forward_prenorm")


def mxfp8_scale_stride(K: int) -> int:
    return 4 * ((K + 127) // 128)


def moe_quantize_mxfp8(x, rows, K, codes, scales, stream=None):
    _check(lib.moe_quantize_mxfp8(_ptr(x), rows, K, _ptr(codes), _ptr(scales), _stream(stream)),
           "moe_quantize_mxfp8")

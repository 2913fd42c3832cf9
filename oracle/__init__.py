"""CPU oracle of the sparse MoE FFN layer -- TEST INFRASTRUCTURE ONLY.

A plain, slow, double-precision C statement of the layer (``moe_ref.c``),
written from the pages that define it, with this thin ctypes wrapper.  Only
``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import it.  The GPU library shares no code with it and never calls
it; the library's Python binding does not import it.

Parity status of each function (how it is pinned to something other than
itself) is listed in the tests under ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_REF_LIB names another build of moe_ref.c to load (the sanitizer test
# builds one with AddressSanitizer and UBSan and runs the oracle's tests on it)
_LIB_PATH = os.environ.get("MOE_REF_LIB") or os.path.join(_HERE, "libmoe_ref.so")

REF_F32, REF_BF16, REF_MXFP4 = 0, 1, 2
REF_SOFTMAX_TOPK, REF_TOPK_SOFTMAX = 0, 1
REF_SWIGLU, REF_SWIGLU_OAI = 0, 1
REF_AQ_NONE, REF_AQ_MXFP8 = 0, 1


def build(force: bool = False) -> str:
    """Compile the oracle with gcc: plain -O2, no fast-math, OpenMP over tokens."""
    src = os.path.join(_HERE, "moe_ref.c")
    hdr = os.path.join(_HERE, "moe_ref.h")
    newest = max(os.path.getmtime(src), os.path.getmtime(hdr))
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < newest:
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class RefMat(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("data", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class RefCfg(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("F", ctypes.c_int32), ("Fs", ctypes.c_int32), ("gating", ctypes.c_int32),
                ("norm_topk_prob", ctypes.c_int32), ("weights_scale", ctypes.c_float),
                ("act", ctypes.c_int32), ("alpha", ctypes.c_float), ("limit", ctypes.c_float),
                ("act_quant", ctypes.c_int32)]


class RefWeights(ctypes.Structure):
    _fields_ = [(n, RefMat) for n in ("router_w", "router_b", "gate_w", "up_w", "gate_up_w",
                                      "gate_up_b", "down_w", "down_b", "sh_gate_w", "sh_up_w",
                                      "sh_down_w", "sh_gate_inp")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        P = ctypes.POINTER
        L.ref_mxfp4_value.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
        L.ref_mxfp4_value.restype = ctypes.c_double
        L.ref_e4m3_value.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
        L.ref_e4m3_value.restype = ctypes.c_double
        L.ref_mxfp8_quantize.argtypes = [vp, ctypes.c_int64, vp, vp]
        L.ref_mxfp8_round.argtypes = [vp, ctypes.c_int64, vp]
        L.ref_elem.argtypes = [P(RefMat), ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
        L.ref_elem.restype = ctypes.c_double
        L.ref_rmsnorm.argtypes = [P(RefMat), i32, i32, P(RefMat), ctypes.c_double, i32, vp]
        L.ref_router_logits.argtypes = [P(RefCfg), P(RefWeights), P(RefMat), i32, vp]
        L.ref_shared_gate_logit.argtypes = [P(RefCfg), P(RefWeights), P(RefMat), i32, vp]
        L.ref_topk.argtypes = [i32, i32, vp, vp]
        L.ref_route.argtypes = [P(RefCfg), vp, i32, vp, vp]
        L.ref_route_prob_key_disagreements.argtypes = [P(RefCfg), vp, i32]
        L.ref_route_prob_key_disagreements.restype = i32
        L.ref_sigmoid.argtypes = [vp, i32, vp]
        L.ref_permute.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp]
        L.ref_expert_act.argtypes = [P(RefCfg), P(RefWeights), i32, vp, vp]
        L.ref_expert_down.argtypes = [P(RefCfg), P(RefWeights), i32, vp, vp]
        L.ref_expert_ffn.argtypes = [P(RefCfg), P(RefWeights), P(RefMat), i32, vp, vp, vp]
        L.ref_combine.argtypes = [P(RefCfg), P(RefWeights), vp, vp, vp, vp, vp, i32, vp]
        L.ref_forward.argtypes = [P(RefCfg), P(RefWeights), P(RefMat), i32, vp, vp, vp, i32,
                                  vp, vp, vp, vp]
        L.ref_forward_dense.argtypes = [P(RefCfg), P(RefWeights), P(RefMat), i32, vp, vp]
        L.ref_set_threads.argtypes = [i32]
        L.ref_set_threads.restype = i32
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


_DT = {"f32": REF_F32, "bf16": REF_BF16, "mxfp4": REF_MXFP4}


def e4m3_value(code: int, e8m0: int = 127) -> float:
    return lib().ref_e4m3_value(code, e8m0)


def mxfp8_quantize(v):
    """float array (last dim a multiple of 32) -> (E4M3 codes uint8, E8M0 scales uint8)."""
    v = np.ascontiguousarray(v, np.float64)
    codes = np.empty(v.shape, np.uint8)
    scales = np.empty(v.shape[:-1] + (v.shape[-1] // 32,), np.uint8)
    lib().ref_mxfp8_quantize(_p(v), v.size, _p(codes), _p(scales))
    return codes, scales


def mxfp8_round(v):
    """float array -> the values its MXFP8 quantisation represents (float64)."""
    v = np.ascontiguousarray(v, np.float64)
    out = np.empty_like(v)
    lib().ref_mxfp8_round(_p(v), v.size, _p(out))
    return out


def rmsnorm(x, g, eps, dtype):
    """RMSNorm of the rows of x ([T][H]) with weight g ([H]) -> the normalised
    rows in `dtype` ('f32': float32, 'bf16': uint16 bf16 bits); x and g are
    given in that same representation."""
    x = np.ascontiguousarray(x)
    g = np.ascontiguousarray(g).reshape(1, -1)
    T, H = x.shape
    out = np.empty((T, H), np.uint16 if dtype == "bf16" else np.float32)
    lib().ref_rmsnorm(ctypes.byref(_mat(x, dtype)), T, H, ctypes.byref(_mat(g, dtype)), float(eps),
                      _DT[dtype], _p(out))
    return out


def _mat(arr, dtype, scales=None):
    if arr is None:
        return RefMat(0, None, None)
    return RefMat(_DT[dtype], _p(arr), _p(scales))


class Layer:
    """Oracle view of a synthetic layer case (keeps its arrays alive)."""

    def __init__(self, case):
        self.case = c = case
        self.cfg = RefCfg(c.H, c.E, c.k, c.F, c.Fs,
                          REF_SOFTMAX_TOPK if c.gating == "softmax_topk" else REF_TOPK_SOFTMAX,
                          int(c.norm_topk_prob), c.weights_scale,
                          REF_SWIGLU if c.act == "swiglu" else REF_SWIGLU_OAI, c.alpha, c.limit,
                          REF_AQ_MXFP8 if getattr(c, "act_quant", "none") == "mxfp8" else REF_AQ_NONE)
        t = c.t
        wd, rd = c.w_dtype, c.router_dtype
        bias_dt = "f32" if wd == "f32" else "bf16"
        w = RefWeights()
        w.router_w = _mat(t.get("router_w"), rd)
        w.router_b = _mat(t.get("router_b"), rd)
        if wd == "mxfp4":
            w.gate_up_w = _mat(t.get("gate_up_codes"), "mxfp4", t.get("gate_up_scales"))
            w.down_w = _mat(t.get("down_codes"), "mxfp4", t.get("down_scales"))
        else:
            w.gate_w = _mat(t.get("gate_w"), wd)
            w.up_w = _mat(t.get("up_w"), wd)
            w.gate_up_w = _mat(t.get("gate_up_w"), wd)
            w.down_w = _mat(t.get("down_w"), wd)
        w.gate_up_b = _mat(t.get("gate_up_b"), bias_dt)
        w.down_b = _mat(t.get("down_b"), bias_dt)
        sd = "f32" if wd == "f32" else "bf16"
        w.sh_gate_w = _mat(t.get("sh_gate_w"), sd)
        w.sh_up_w = _mat(t.get("sh_up_w"), sd)
        w.sh_down_w = _mat(t.get("sh_down_w"), sd)
        w.sh_gate_inp = _mat(t.get("sh_gate_inp"), sd)
        self.w = w
        self.x = _mat(t["x"], c.x_dtype)

    def with_x(self, x):
        """A RefMat for another activation array of the case's dtype."""
        return _mat(x, self.case.x_dtype)

    # -- steps
    def router_logits(self, T=None):
        T = self.case.T if T is None else T
        out = np.empty((T, self.case.E), np.float32)
        lib().ref_router_logits(ctypes.byref(self.cfg), ctypes.byref(self.w), ctypes.byref(self.x), T, _p(out))
        return out

    def shared_gate_logit(self):
        out = np.empty(self.case.T, np.float32)
        lib().ref_shared_gate_logit(ctypes.byref(self.cfg), ctypes.byref(self.w), ctypes.byref(self.x),
                                    self.case.T, _p(out))
        return out

    def route(self, logits):
        logits = np.ascontiguousarray(logits, np.float32)
        T = logits.shape[0]
        idx = np.empty((T, self.case.k), np.int32)
        wt = np.empty((T, self.case.k), np.float32)
        lib().ref_route(ctypes.byref(self.cfg), _p(logits), T, _p(idx), _p(wt))
        return idx, wt

    def prob_key_disagreements(self, logits):
        logits = np.ascontiguousarray(logits, np.float32)
        return lib().ref_route_prob_key_disagreements(ctypes.byref(self.cfg), _p(logits), logits.shape[0])

    def expert_act(self, e, xrow):
        xrow = np.ascontiguousarray(xrow, np.float64)
        n = self.case.Fs if e == self.case.E else self.case.F
        h = np.empty(n, np.float64)
        lib().ref_expert_act(ctypes.byref(self.cfg), ctypes.byref(self.w), e, _p(xrow), _p(h))
        return h

    def expert_down(self, e, h):
        h = np.ascontiguousarray(h, np.float64)
        y = np.empty(self.case.H, np.float64)
        lib().ref_expert_down(ctypes.byref(self.cfg), ctypes.byref(self.w), e, _p(h), _p(y))
        return y

    def expert_ffn(self, offsets, sorted_assign):
        c = self.case
        offsets = np.ascontiguousarray(offsets, np.int32)
        sorted_assign = np.ascontiguousarray(sorted_assign, np.int32)
        nseg = c.E + (1 if c.has_shared else 0)
        n = c.T * c.k
        assert int(offsets[nseg]) == n + (c.T if c.has_shared else 0)
        # routed rows (F values each) first, then the shared rows (Fs values)
        h = np.empty(n * c.F + (c.T * c.Fs if c.has_shared else 0), np.float32)
        lib().ref_expert_ffn(ctypes.byref(self.cfg), ctypes.byref(self.w), ctypes.byref(self.x), c.T,
                             _p(offsets), _p(sorted_assign), _p(h))
        return h

    def combine(self, h, offsets, sorted_assign, topk_w, sgate):
        c = self.case
        h = np.ascontiguousarray(h, np.float32)
        out = np.empty((c.T, c.H), np.float32)
        sg = None if sgate is None else np.ascontiguousarray(sgate, np.float32)
        lib().ref_combine(ctypes.byref(self.cfg), ctypes.byref(self.w), _p(h),
                          _p(np.ascontiguousarray(offsets, np.int32)),
                          _p(np.ascontiguousarray(sorted_assign, np.int32)),
                          _p(np.ascontiguousarray(topk_w, np.float32)), _p(sg), c.T, _p(out))
        return out

    def forward(self, logits=None, idx=None, tokens=None):
        """Whole layer; returns (out, topk_idx, topk_w, sgate).  With `tokens`,
        only those rows are computed (the others are left as NaN)."""
        c = self.case
        out = np.full((c.T, c.H), np.nan, np.float32)
        ti = np.full((c.T, c.k), -1, np.int32)
        tw = np.full((c.T, c.k), np.nan, np.float32)
        sg = np.full(c.T, np.nan, np.float32)
        lg = None if logits is None else np.ascontiguousarray(logits, np.float32)
        ix = None if idx is None else np.ascontiguousarray(idx, np.int32)
        tk = None if tokens is None else np.ascontiguousarray(tokens, np.int32)
        lib().ref_forward(ctypes.byref(self.cfg), ctypes.byref(self.w), ctypes.byref(self.x), c.T,
                          _p(lg), _p(ix), _p(tk), 0 if tk is None else len(tk),
                          _p(out), _p(ti), _p(tw), _p(sg))
        return out, ti, tw, sg

    def block_forward(self, tokens=None, logits=None, idx=None):
        """The layer inside its decoder block: out = r + layer(RMSNorm(r) * g)
        with r = the case's "resid" rows, g its "norm_w", eps its norm_eps.
        Returns (out, xn, topk_idx, topk_w, sgate); the residual sum is taken
        in double from the layer's fp32 output and rounded to fp32.  With
        `idx`, the layer takes those picks instead of routing."""
        c = self.case
        xn = rmsnorm(c.t["resid"], c.t["norm_w"], c.norm_eps, c.x_dtype)
        keep = self.x
        self._xn = xn
        self.x = _mat(xn, c.x_dtype)
        try:
            out, ti, tw, sg = self.forward(logits=logits, idx=idx, tokens=tokens)
        finally:
            self.x = keep
        r = c.t["resid"]
        r = (bf16_to_f64(r) if c.x_dtype == "bf16" else np.asarray(r, np.float64))
        out = (r + out.astype(np.float64)).astype(np.float32)
        return out, xn, ti, tw, sg

    def forward_dense(self, logits=None):
        c = self.case
        out = np.empty((c.T, c.H), np.float64)
        lg = None if logits is None else np.ascontiguousarray(logits, np.float32)
        lib().ref_forward_dense(ctypes.byref(self.cfg), ctypes.byref(self.w), ctypes.byref(self.x), c.T,
                                _p(lg), _p(out))
        return out


def bf16_to_f64(b):
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def topk(keys, k):
    keys = np.ascontiguousarray(keys, np.float32)
    idx = np.empty(k, np.int32)
    lib().ref_topk(len(keys), k, _p(keys), _p(idx))
    return idx


def sigmoid(s):
    s = np.ascontiguousarray(s, np.float32).ravel()
    out = np.empty_like(s)
    lib().ref_sigmoid(_p(s), len(s), _p(out))
    return out


def permute(E, k, T, shared, topk_idx):
    topk_idx = np.ascontiguousarray(topk_idx, np.int32)
    n = T * k + (T if shared else 0)
    offsets = np.empty(E + 1 + (1 if shared else 0), np.int32)
    sa = np.empty(max(n, 1), np.int32)
    ap = np.empty(max(n, 1), np.int32)
    lib().ref_permute(E, k, T, int(shared), _p(topk_idx), _p(offsets), _p(sa), _p(ap))
    return offsets, sa[:n], ap[:n]


def set_threads(n: int) -> int:
    """Threads of the oracle's parallel loops (0: unchanged); returns the count."""
    return lib().ref_set_threads(n)


def mxfp4_value(code, e8m0):
    return lib().ref_mxfp4_value(code, e8m0)

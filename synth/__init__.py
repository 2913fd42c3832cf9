"""Seeded synthetic inputs for the sparse MoE FFN layer.

This package is shared by the CPU oracle's tests, the GPU library's tests and
the benchmark.  It draws numbers and lays them out in the shapes of the
layers the pages describe; it contains none of the layer's arithmetic
(no dot products, gating, activations or combines).

Recipe (see ``synth.c`` for the draw mappings):

* every tensor row is its own xorshift32 stream, id ``(tensor_id << 32) + row``,
  base seed 0x9E3779B9 (the seed the qwen35moe golden-vector page names);
* activations ~ N(0, 1); weights ~ N(0, 1/fan_in) with fan_in the input width
  of the matrix (H for router, gate, up, gate_up and the shared gate; F for
  down); biases ~ N(0, 1/fan_in) as well;
* bf16 tensors are the fp32 draws rounded to nearest even;
* MXFP4 codes are uniform random bytes (two E2M1 codes per byte), E8M0 block
  exponents uniform in [118, 130];
* the prefill-sized qwen35moe-shaped layer takes router logits drawn from a
  Zipf(1.0)-over-experts Gumbel model instead of a router product.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
BASE_SEED = 0x9E3779B9

# Tensor ids (stream id = tensor_id << 32 | row).
TID = {
    "x": 1, "router_w": 2, "router_b": 3, "gate_w": 4, "up_w": 5, "gate_up_w": 6,
    "gate_up_b": 7, "down_w": 8, "down_b": 9, "sh_gate_w": 10, "sh_up_w": 11,
    "sh_down_w": 12, "sh_gate_inp": 13, "gate_up_codes": 14, "gate_up_scales": 15,
    "down_codes": 16, "down_scales": 17, "logits": 18, "resid": 19, "norm_w": 20,
    "resid_scale": 21,
}


def build(force: bool = False) -> str:
    """Compile ``libsynth.so`` with gcc (plain -O2, OpenMP over rows)."""
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        u32, u64, i64, i32, dbl, vp = (ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int64,
                                       ctypes.c_int32, ctypes.c_double, ctypes.c_void_p)
        L.synth_stream_seed.argtypes = [u32, u64]; L.synth_stream_seed.restype = u32
        L.synth_xorshift32_next.argtypes = [u32]; L.synth_xorshift32_next.restype = u32
        L.synth_f32_to_bf16.argtypes = [ctypes.c_float]; L.synth_f32_to_bf16.restype = ctypes.c_uint16
        L.synth_normal_f32.argtypes = [u32, u64, dbl, i64, i64, vp]
        L.synth_normal_bf16.argtypes = [u32, u64, dbl, i64, i64, vp]
        L.synth_bytes.argtypes = [u32, u64, i64, i64, vp]
        L.synth_range_bytes.argtypes = [u32, u64, i64, i64, u32, u32, vp]
        L.synth_permutation.argtypes = [u32, u64, i32, vp]
        L.synth_zipf_logits.argtypes = [u32, u64, i32, i32, dbl, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def normal(tensor: str, shape, std: float, dtype: str, seed: int = BASE_SEED) -> np.ndarray:
    """N(0, std^2) draws; dtype 'f32' -> float32, 'bf16' -> uint16 bf16 bits."""
    shape = tuple(int(s) for s in shape)
    cols = shape[-1] if shape else 1
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    if dtype == "f32":
        out = np.empty(shape, dtype=np.float32)
        if out.size:
            lib().synth_normal_f32(seed, TID[tensor] << 32, std, rows, cols, _ptr(out))
    elif dtype == "bf16":
        out = np.empty(shape, dtype=np.uint16)
        if out.size:
            lib().synth_normal_bf16(seed, TID[tensor] << 32, std, rows, cols, _ptr(out))
    else:
        raise ValueError(dtype)
    return out


def random_bytes(tensor: str, shape, seed: int = BASE_SEED) -> np.ndarray:
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint8)
    if out.size:
        lib().synth_bytes(seed, TID[tensor] << 32, int(np.prod(shape[:-1])), shape[-1], _ptr(out))
    return out


def range_bytes(tensor: str, shape, lo: int, span: int, seed: int = BASE_SEED) -> np.ndarray:
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint8)
    if out.size:
        lib().synth_range_bytes(seed, TID[tensor] << 32, int(np.prod(shape[:-1])), shape[-1], lo, span, _ptr(out))
    return out


def zipf_logits(T: int, E: int, exponent: float = 1.0, seed: int = BASE_SEED) -> np.ndarray:
    out = np.empty((T, E), dtype=np.float32)
    lib().synth_zipf_logits(seed, TID["logits"] << 32, T, E, exponent, _ptr(out))
    return out


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even (storage conversion only)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# Layer cases

@dataclass
class Case:
    """One synthetic MoE layer: shape/config fields plus its tensors (numpy)."""
    name: str
    T: int
    H: int
    E: int
    k: int
    F: int
    Fs: int                      # shared expert FF width, 0 = none
    gating: str                  # "softmax_topk" (qwen) | "topk_softmax" (gpt-oss)
    norm_topk_prob: bool
    weights_scale: float
    act: str                     # "swiglu" | "swiglu_oai"
    alpha: float
    limit: float
    x_dtype: str                 # "f32" | "bf16"
    w_dtype: str                 # "f32" | "bf16" | "mxfp4"
    router_dtype: str            # "f32" | "bf16"
    drawn_logits: bool = False   # logits are an input; no router product
    act_quant: str = "none"      # "none" | "mxfp8": routed experts' GEMM inputs rounded to MXFP8
    norm_eps: float = 1e-6       # RMSNorm epsilon of the block around the layer
    t: dict = field(default_factory=dict)

    @property
    def has_shared(self) -> bool:
        return self.Fs > 0


def _tiny_case(T: int = 8, seed: int = BASE_SEED, only=None) -> Case:
    """fp32 layer small enough for brute force, with planted exact ties.

    Router rows 9 and 13 are copies of row 4, row 12 a copy of row 7, so those
    experts' logits are bit-equal for every token.  Token 3 is a multiple of
    router row 4 (experts 4, 9, 13 tie at the top, first-seen picks 4 then 9);
    token 6 is 2*row0 + row7 (expert 0 first, 7 and 12 tie for second).
    """
    H, E, k, F, Fs = 256, 16, 2, 128, 128
    c = Case("tiny_fp32", T, H, E, k, F, Fs, "softmax_topk", True, 1.0, "swiglu", 1.702, 7.0,
             "f32", "f32", "f32")
    x = normal("x", (T, H), 1.0, "f32", seed)
    wr = normal("router_w", (E, H), 1.0 / np.sqrt(H), "f32", seed)
    wr[9] = wr[4]
    wr[13] = wr[4]
    wr[12] = wr[7]
    if T > 3:
        x[3] = np.float32(16.0) * wr[4]
    if T > 6:
        x[6] = np.float32(32.0) * wr[0] + np.float32(16.0) * wr[7]
    c.t["x"] = x
    c.t["router_w"] = wr
    c.t["gate_w"] = normal("gate_w", (E, F, H), 1.0 / np.sqrt(H), "f32", seed)
    c.t["up_w"] = normal("up_w", (E, F, H), 1.0 / np.sqrt(H), "f32", seed)
    c.t["down_w"] = normal("down_w", (E, H, F), 1.0 / np.sqrt(F), "f32", seed)
    c.t["sh_gate_w"] = normal("sh_gate_w", (Fs, H), 1.0 / np.sqrt(H), "f32", seed)
    c.t["sh_up_w"] = normal("sh_up_w", (Fs, H), 1.0 / np.sqrt(H), "f32", seed)
    c.t["sh_down_w"] = normal("sh_down_w", (H, Fs), 1.0 / np.sqrt(Fs), "f32", seed)
    c.t["sh_gate_inp"] = normal("sh_gate_inp", (1, H), 1.0 / np.sqrt(H), "f32", seed)[0]
    return c


def _qwen_case(T: int, drawn: bool, seed: int = BASE_SEED, E: int = 256, H: int = 2048,
               F: int = 512, Fs: int = 512, k: int = 8, only=None) -> Case:
    name = "qwen35moe_prefill_zipf" if drawn else "qwen35moe_decode"
    c = Case(name, T, H, E, k, F, Fs, "softmax_topk", True, 1.0, "swiglu", 1.702, 7.0,
             "bf16", "bf16", "bf16", drawn_logits=drawn)
    want = (lambda n: True) if only is None else (lambda n: n in only)
    if want("x"):
        c.t["x"] = normal("x", (T, H), 1.0, "bf16", seed)
    if want("router_w"):
        c.t["router_w"] = normal("router_w", (E, H), 1.0 / np.sqrt(H), "bf16", seed)
    if want("gate_w"):
        c.t["gate_w"] = normal("gate_w", (E, F, H), 1.0 / np.sqrt(H), "bf16", seed)
    if want("up_w"):
        c.t["up_w"] = normal("up_w", (E, F, H), 1.0 / np.sqrt(H), "bf16", seed)
    if want("down_w"):
        c.t["down_w"] = normal("down_w", (E, H, F), 1.0 / np.sqrt(F), "bf16", seed)
    if want("sh_gate_w"):
        c.t["sh_gate_w"] = normal("sh_gate_w", (Fs, H), 1.0 / np.sqrt(H), "bf16", seed)
    if want("sh_up_w"):
        c.t["sh_up_w"] = normal("sh_up_w", (Fs, H), 1.0 / np.sqrt(H), "bf16", seed)
    if want("sh_down_w"):
        c.t["sh_down_w"] = normal("sh_down_w", (H, Fs), 1.0 / np.sqrt(Fs), "bf16", seed)
    if want("sh_gate_inp"):
        c.t["sh_gate_inp"] = normal("sh_gate_inp", (1, H), 1.0 / np.sqrt(H), "bf16", seed)[0]
    if drawn and want("logits"):
        c.t["logits"] = zipf_logits(T, E, 1.0, seed)
    return c


def _gptoss_case(T: int, mxfp4: bool, seed: int = BASE_SEED, E: int = 32, H: int = 2880,
                 F: int = 2880, k: int = 4, Fs: int = 0, only=None) -> Case:
    """gpt-oss-shaped layer; Fs > 0 adds a (bf16, plain SwiGLU) shared expert,
    which the pages do not give gpt-oss but the boundary allows for any layer."""
    name = "gptoss20b_mxfp4" if mxfp4 else "gptoss20b_bf16"
    c = Case(name, T, H, E, k, F, Fs, "topk_softmax", False, 1.0, "swiglu_oai", 1.702, 7.0,
             "bf16", "mxfp4" if mxfp4 else "bf16", "bf16")
    want = (lambda n: True) if only is None else (lambda n: n in only)
    if want("x"):
        c.t["x"] = normal("x", (T, H), 1.0, "bf16", seed)
    if want("router_w"):
        c.t["router_w"] = normal("router_w", (E, H), 1.0 / np.sqrt(H), "bf16", seed)
        c.t["router_b"] = normal("router_b", (1, E), 1.0 / np.sqrt(H), "bf16", seed)[0]
    if not want("experts"):
        return c
    c.t["gate_up_b"] = normal("gate_up_b", (E, 2 * F), 1.0 / np.sqrt(H), "bf16", seed)
    c.t["down_b"] = normal("down_b", (E, H), 1.0 / np.sqrt(F), "bf16", seed)
    if mxfp4:
        c.t["gate_up_codes"] = random_bytes("gate_up_codes", (E, 2 * F, H // 32, 16), seed)
        c.t["gate_up_scales"] = range_bytes("gate_up_scales", (E, 2 * F, H // 32), 118, 13, seed)
        c.t["down_codes"] = random_bytes("down_codes", (E, H, F // 32, 16), seed)
        c.t["down_scales"] = range_bytes("down_scales", (E, H, F // 32), 118, 13, seed)
    else:
        c.t["gate_up_w"] = normal("gate_up_w", (E, 2 * F, H), 1.0 / np.sqrt(H), "bf16", seed)
        c.t["down_w"] = normal("down_w", (E, H, F), 1.0 / np.sqrt(F), "bf16", seed)
    if Fs > 0:
        c.t["sh_gate_w"] = normal("sh_gate_w", (Fs, H), 1.0 / np.sqrt(H), "bf16", seed)
        c.t["sh_up_w"] = normal("sh_up_w", (Fs, H), 1.0 / np.sqrt(H), "bf16", seed)
        c.t["sh_down_w"] = normal("sh_down_w", (H, Fs), 1.0 / np.sqrt(Fs), "bf16", seed)
        c.t["sh_gate_inp"] = normal("sh_gate_inp", (1, H), 1.0 / np.sqrt(H), "bf16", seed)[0]
    return c


CASES = {
    # name: (builder, default T)
    "tiny_fp32": (lambda T, **kw: _tiny_case(T, **kw), 8),
    "qwen35moe_decode": (lambda T, **kw: _qwen_case(T, False, **kw), 8),
    "qwen35moe_prefill_zipf": (lambda T, **kw: _qwen_case(T, True, **kw), 4096),
    "gptoss20b_bf16": (lambda T, **kw: _gptoss_case(T, False, **kw), 2048),
    "gptoss20b_mxfp4": (lambda T, **kw: _gptoss_case(T, True, **kw), 2048),
}


def add_block_inputs(c: Case, seed: int = BASE_SEED) -> Case:
    """Inputs of the decoder block around the layer: the residual stream
    "resid" [T][H] (N(0,1) rows times a per-token power of two in
    2^-3..2^4, so every token has its own RMS) and the norm weight "norm_w"
    [H], 1 + N(0, 0.1^2) (norm weights centred near 1), both in the case's
    activation dtype; norm_eps is the model's (gpt-oss 1e-5, qwen35moe
    1e-6).  The layer's own "x" is left as it is."""
    T, H = c.T, c.H
    scale = 2.0 ** (range_bytes("resid_scale", (1, max(T, 1)), 0, 8, seed)[0, :T].astype(np.float32) - 3.0)
    r = normal("resid", (T, H), 1.0, "f32", seed) * scale[:, None]
    g = normal("norm_w", (1, H), 0.1, "f32", seed)[0] + np.float32(1.0)
    if c.x_dtype == "bf16":
        r, g = bf16_bits(r), bf16_bits(g)
    c.t["resid"] = np.ascontiguousarray(r)
    c.t["norm_w"] = np.ascontiguousarray(g)
    c.norm_eps = 1e-5 if c.gating == "topk_softmax" else 1e-6
    return c


def make_case(name: str, T: int | None = None, **kw) -> Case:
    builder, t_default = CASES[name]
    return builder(t_default if T is None else T, **kw)


from . import vecfile  # noqa: E402  (self-describing vector files and the on-disk case cache)

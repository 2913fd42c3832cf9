"""CPU-side checks of the C-ABI library: it loads, it exports every entry
point include/moe.h declares, and its host-side argument validation returns
the documented status codes before launching anything (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    assert _declared() == sorted(["moe_workspace_bytes", "moe_route", "moe_permute", "moe_expert_ffn",
                                  "moe_combine", "moe_forward", "moe_forward_noalloc", "moe_forward_prenorm",
                                  "moe_quantize_mxfp8",
                                  "moe_status_string"])


def test_library_exports_every_declared_symbol():
    import sparse_moe_ffn_router_amd as moe
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (moe_[a-z0-9_]+)$", out, flags=re.M))
    for name in _declared():
        assert name in exported, name
        assert getattr(moe.lib, name) is not None
    assert set(moe.EXPORTS) == set(_declared())


def _cfg(**kw):
    import sparse_moe_ffn_router_amd as moe
    base = dict(hidden=2048, n_expert=256, top_k=8, expert_ff=512, shared_ff=512)
    base.update(kw)
    return moe.MoeConfig(**base)


def test_workspace_bytes_and_config_validation():
    import sparse_moe_ffn_router_amd as moe
    assert moe.moe_workspace_bytes(_cfg(), 8) > 0
    assert moe.moe_workspace_bytes(_cfg(), 4096) > moe.moe_workspace_bytes(_cfg(), 8)
    # y rows (fp32) dominate at prefill size: (T*k + T) * H * 4 bytes
    assert moe.moe_workspace_bytes(_cfg(), 4096) >= (4096 * 9) * 2048 * 4
    for bad in (dict(top_k=0), dict(top_k=300), dict(n_expert=2048, top_k=8), dict(hidden=-1),
                dict(gating=7), dict(act=9), dict(x_dtype=5)):
        assert moe.moe_workspace_bytes(_cfg(**bad), 8) == 0, bad
    for unsup in (dict(hidden=2050), dict(expert_ff=500), dict(x_dtype=moe.DTYPE_F32),
                  dict(w_dtype=moe.DTYPE_MXFP4)):  # mxfp4 needs the interleaved gate_up layout
        assert moe.moe_workspace_bytes(_cfg(**unsup), 8) == 0, unsup


def test_act_quant_validation():
    import sparse_moe_ffn_router_amd as moe
    mx = dict(hidden=2880, n_expert=32, top_k=4, expert_ff=2880, shared_ff=0, gating=moe.GATING_TOPK_SOFTMAX,
              norm_topk_prob=False, act=moe.ACT_SWIGLU_OAI, w_dtype=moe.DTYPE_MXFP4)
    plain = moe.moe_workspace_bytes(_cfg(**mx), 2048)
    quant = moe.moe_workspace_bytes(_cfg(act_quant=moe.ACT_QUANT_MXFP8, **mx), 2048)
    assert plain > 0 and quant > plain
    # rounded x and h (2 bytes per element) plus their scale words
    assert quant - plain >= 2048 * 2880 * 2 + 2048 * 4 * 2880 * 2
    assert moe.moe_workspace_bytes(_cfg(act_quant=7, **mx), 8) == 0
    for unsup in (dict(w_dtype=moe.DTYPE_BF16), dict(shared_ff=512), dict(hidden=2880 + 32),
                  dict(expert_ff=2880 - 32)):
        c = dict(mx)
        c.update(unsup)
        assert moe.moe_workspace_bytes(_cfg(act_quant=moe.ACT_QUANT_MXFP8, **c), 64) == 0, unsup


def test_quantize_argument_checks():
    import sparse_moe_ffn_router_amd as moe
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    q = moe.lib.moe_quantize_mxfp8
    fake = vp(1 << 20)
    assert q(fake, i64(4), i32(48), fake, fake, None) == moe.MOE_EINVAL     # K not a multiple of 32
    assert q(None, i64(4), i32(64), fake, fake, None) == moe.MOE_EINVAL     # null input
    assert q(vp((1 << 20) + 2), i64(4), i32(64), fake, fake, None) == moe.MOE_EINVAL  # misaligned
    assert q(fake, i64(-1), i32(64), fake, fake, None) == moe.MOE_EINVAL
    assert q(None, i64(0), i32(64), None, None, None) == moe.MOE_OK          # no rows: nothing to do


def _raw(fn, *args):
    import sparse_moe_ffn_router_amd as moe
    return getattr(moe.lib, fn)(*args)


def test_entry_points_reject_bad_arguments_before_launch():
    import sparse_moe_ffn_router_amd as moe
    c = _cfg()._c()
    W = moe._Weights()
    cb = ctypes.byref(c)
    wb = ctypes.byref(W)
    # T = 0 is a no-op everywhere
    assert _raw("moe_expert_ffn", cb, wb, None, None, None, 0, None, None, 0, None) == moe.MOE_EINVAL  # no weights
    fake = 1 << 20  # never dereferenced: every call below fails its host checks first
    full = moe._Weights(*([fake] * len(moe._WEIGHT_FIELDS)))
    fb = ctypes.byref(full)
    assert _raw("moe_expert_ffn", cb, fb, None, None, None, 0, None, None, 0, None) == moe.MOE_OK
    assert _raw("moe_route", cb, fb, None, None, None, None, None, 0, None, 0, None) == moe.MOE_OK
    assert _raw("moe_permute", cb, None, 0, None, None, None, None, 0, None) == moe.MOE_OK
    # negative T
    assert _raw("moe_route", cb, fb, None, None, None, None, None, -1, None, 0, None) == moe.MOE_EINVAL
    # missing outputs
    assert _raw("moe_route", cb, fb, fake, None, fake, fake, fake, 8, None, 0, None) == moe.MOE_EINVAL
    # shared expert needs sgate
    assert _raw("moe_route", cb, fb, fake, fake, fake, fake, None, 8, None, 0, None) == moe.MOE_EINVAL
    # misaligned pointer
    assert _raw("moe_route", cb, fb, fake + 2, fake, fake, fake, fake, 8, None, 0, None) == moe.MOE_EINVAL
    # route scratch: optional, but when given at least moe_workspace_bytes
    assert _raw("moe_route", cb, fb, fake, fake, fake, fake, fake, 4096, fake, 16, None) == moe.MOE_EWORKSPACE
    mis = moe._Weights(*([fake] * len(moe._WEIGHT_FIELDS)))
    mis.gate_w = fake + 4
    assert _raw("moe_expert_ffn", cb, ctypes.byref(mis), fake, fake, fake, 8, fake, None, 0, None) == moe.MOE_EINVAL
    # workspace too small / misaligned
    assert _raw("moe_combine", cb, fb, fake, fake, fake, fake, fake, 8, fake, fake, 16, None) == moe.MOE_EWORKSPACE
    need = moe.moe_workspace_bytes(_cfg(), 4096)
    assert _raw("moe_forward", cb, fb, fake, 4096, fake, None, None, None, None, fake, need - 1, None) == moe.MOE_EWORKSPACE
    assert _raw("moe_forward", cb, fb, fake, 4096, fake, None, None, None, None, fake + 64, need, None) == moe.MOE_EWORKSPACE
    assert _raw("moe_permute", cb, fake, 4096, fake, fake, fake, None, 0, None) == moe.MOE_EWORKSPACE
    # drawn logits (no router) need the logits buffer
    nr = moe._Weights(*([fake] * len(moe._WEIGHT_FIELDS)))
    nr.router_w = None
    assert _raw("moe_forward", cb, ctypes.byref(nr), fake, 8, fake, None, None, None, None, fake, need, None) == moe.MOE_EINVAL
    # the pre-norm block: norm weight, residual and a sane eps are required
    pre = lambda nw, eps, r, T, out, xn, ws, nb: _raw("moe_forward_prenorm", cb, fb, nw, ctypes.c_float(eps), r, T,
                                                      out, xn, None, None, None, None, ws, nb, None)
    assert pre(None, 1e-6, None, 0, None, None, None, 0) == moe.MOE_OK                   # T = 0
    assert pre(None, 1e-6, fake, 8, fake, None, fake, need) == moe.MOE_EINVAL          # no norm weight
    assert pre(fake, 1e-6, None, 8, fake, None, fake, need) == moe.MOE_EINVAL          # no residual
    assert pre(fake, -1.0, fake, 8, fake, None, fake, need) == moe.MOE_EINVAL          # negative eps
    assert pre(fake, float("nan"), fake, 8, fake, None, fake, need) == moe.MOE_EINVAL  # NaN eps
    assert pre(fake, 1e-6, fake + 8, 8, fake, None, fake, need) == moe.MOE_EINVAL      # misaligned residual
    assert pre(fake, 1e-6, fake, 8, fake, fake + 2, fake, need) == moe.MOE_EINVAL      # misaligned xn
    assert pre(fake, 1e-6, fake, 4096, fake, None, fake, need - 1) == moe.MOE_EWORKSPACE
    # unsupported combination
    c2 = _cfg(w_dtype=moe.DTYPE_MXFP4)._c()
    assert _raw("moe_route", ctypes.byref(c2), fb, fake, fake, fake, fake, fake, 8, None, 0, None) == moe.MOE_EUNSUPPORTED


def test_status_strings():
    import sparse_moe_ffn_router_amd as moe
    for s in (moe.MOE_OK, moe.MOE_EINVAL, moe.MOE_EUNSUPPORTED, moe.MOE_EWORKSPACE, moe.MOE_EHIP):
        assert moe.status_string(s) and moe.status_string(s) != "unknown status"
    assert moe.status_string(12345) == "unknown status"


def test_batches_past_32_bit_buffer_extents_are_rejected():
    """The kernels address the token rows (and, on the MX MFMA path, the
    MXFP8 codes of h) through buffer descriptors with 32-bit extents; a batch
    whose rows would pass 2 GiB is refused on the host (no workspace size,
    MOE_EUNSUPPORTED from the entry points) instead of wrapping."""
    import sparse_moe_ffn_router_amd as moe
    T_max = (2 ** 31 - 1) // (2048 * 2)            # bf16 x rows of H = 2048 just below 2 GiB
    assert moe.moe_workspace_bytes(_cfg(), T_max) > 0
    assert moe.moe_workspace_bytes(_cfg(), T_max + 1) == 0
    fake = 1 << 20
    wb = moe._Weights(*([fake] * len(moe._WEIGHT_FIELDS)))
    cb = _cfg()._c()
    assert _raw("moe_forward", ctypes.byref(cb), ctypes.byref(wb), fake, T_max + 1, fake, None, None, None, None,
                fake, 1 << 40, None) == moe.MOE_EUNSUPPORTED
    mx = dict(hidden=2880, n_expert=32, top_k=4, expert_ff=2880, shared_ff=0, gating=moe.GATING_TOPK_SOFTMAX,
              act=moe.ACT_SWIGLU_OAI, w_dtype=moe.DTYPE_MXFP4, act_quant=moe.ACT_QUANT_MXFP8)
    T_h = (2 ** 31 - 1) // (4 * 2880)             # E4M3 codes of h: T*k*F bytes
    assert moe.moe_workspace_bytes(_cfg(**mx), T_h) > 0
    assert moe.moe_workspace_bytes(_cfg(**mx), T_h + 1) == 0

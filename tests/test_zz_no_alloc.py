"""The allocation-free entry point (moe_forward_noalloc, built-in scratch)
against moe_forward with a caller's workspace: the same kernels on the same
inputs, so outputs, logits, picks, weights and the shared gate must be
bit-identical -- on two calls in a row, the second with a smaller batch (the
scratch keeps the first call's contents), and a batch too large for the
scratch is refused."""
import numpy as np
import pytest
import torch

import sparse_moe_ffn_router_amd as moe
import synth
from tests._gpu import config_of, device_weights, to_torch
from tests._parity import log

pytestmark = pytest.mark.gpu


def _outputs(case, T):
    return dict(out=torch.full((T, case.H), float("nan"), dtype=torch.float32, device="cuda"),
                logits=torch.full((T, case.E), float("nan"), dtype=torch.float32, device="cuda"),
                topk_idx=torch.full((T, case.k), -1, dtype=torch.int32, device="cuda"),
                topk_w=torch.full((T, case.k), float("nan"), dtype=torch.float32, device="cuda"),
                sgate=torch.full((T,), float("nan"), dtype=torch.float32, device="cuda") if case.has_shared else None)


def _both(case, w, x, T):
    cfg = config_of(case)
    a, b = _outputs(case, T), _outputs(case, T)
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    moe.moe_forward(cfg, w, x, T, a["out"], ws, logits=a["logits"], topk_idx=a["topk_idx"], topk_w=a["topk_w"],
                    sgate=a["sgate"])
    moe.moe_forward_noalloc(cfg, w, x, T, b["out"], logits=b["logits"], topk_idx=b["topk_idx"],
                            topk_w=b["topk_w"], sgate=b["sgate"])
    torch.cuda.synchronize()
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), "%s differs (T=%d)" % (k, T)


@pytest.mark.parametrize("name,over,T1,T2", [
    ("qwen35moe_decode", {}, 64, 8),                                   # decode layer, then a smaller batch
    ("gptoss20b_mxfp4", {}, 16, 3),                                    # MXFP4 few-token path
    ("qwen35moe_decode", dict(E=16, H=256, F=192, Fs=128, k=4), 300, 40),   # MFMA tiles, then the GEMV path
])
def test_noalloc_matches_moe_forward_on_two_calls(name, over, T1, T2):
    log("noalloc %s T=%d then T=%d" % (name, T1, T2))
    case = synth.make_case(name, T=T1, **over)
    w = device_weights(case)
    x = to_torch(case.t["x"])
    _both(case, w, x, T1)
    _both(case, w, x[:T2].contiguous(), T2)


def test_noalloc_refuses_batches_past_its_scratch():
    case = synth.make_case("qwen35moe_decode", T=8)
    cfg = config_of(case)
    T = 8
    while moe.moe_workspace_bytes(cfg, T) <= moe.NOALLOC_SCRATCH_BYTES:
        T *= 2
    w = device_weights(case)
    x = torch.zeros((T, case.H), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((T, case.H), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward_noalloc(cfg, w, x, T, out)
    assert ei.value.status == moe.MOE_EWORKSPACE

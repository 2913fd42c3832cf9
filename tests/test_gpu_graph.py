"""moe_forward captured in a HIP graph and replayed.

The library neither allocates, frees, synchronises nor clears memory with
memset, so a whole layer pass can be captured once and replayed.  Each case
replays the graph several times, with new token contents copied into the
captured input and eager layer passes run between the replays, and checks
every replay bit for bit against an eager pass on the same input (the same
kernels on the same data give the same bits), and the first one against the
oracle."""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_ffn_router_amd as moe
import synth
from tests._gpu import config_of, device_weights, to_torch
from tests._parity import assert_normwise, log, tol_of

pytestmark = pytest.mark.gpu

CASES = [
    ("qwen35moe_decode", 8, dict(E=32, H=256, F=128, Fs=128, k=4)),   # few-token kernels
    ("qwen35moe_decode", 300, dict(E=16, H=256, F=192, Fs=128, k=4)),  # MFMA tiles, multi-launch permutation
    ("gptoss20b_mxfp4", 16, dict(E=8, H=320, F=192, k=2)),            # MXFP4 burst kernels
    ("gptoss20b_mxfp4", 150, dict(E=8, H=320, F=192, k=2)),           # MXFP4 MFMA tiles
]


def _ids(p):
    return "%s-T%d" % (p[0], p[1])


@pytest.mark.parametrize("name,T,over", CASES, ids=[_ids(p) for p in CASES])
def test_forward_graph_replay(name, T, over):
    log("graph replay: %s T=%d %s" % (name, T, over))
    case = synth.make_case(name, T=T, **over)
    cfg = config_of(case)
    w = device_weights(case)
    xs = [case.t["x"]] + [synth.make_case(name, T=T, seed=synth.BASE_SEED + i, only={"x"}, **over).t["x"]
                          for i in (1, 2, 3)]
    x_static = to_torch(xs[0])
    out_g = torch.empty((T, case.H), dtype=torch.float32, device="cuda")
    idx_g = torch.empty((T, case.k), dtype=torch.int32, device="cuda")
    ws_g = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    out_e = torch.empty_like(out_g)
    idx_e = torch.empty_like(idx_g)
    ws_e = torch.empty_like(ws_g)

    # warm the launch path on a side stream before capturing
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.moe_forward(cfg, w, x_static, T, out_g, ws_g, topk_idx=idx_g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_forward(cfg, w, x_static, T, out_g, ws_g, topk_idx=idx_g)
    torch.cuda.synchronize()

    for rep, xn in enumerate(xs):
        x_static.copy_(to_torch(xn))
        out_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        moe.moe_forward(cfg, w, to_torch(xn), T, out_e, ws_e, topk_idx=idx_e)
        torch.cuda.synchronize()
        assert torch.equal(idx_g, idx_e), "replay %d: routing differs from the eager pass" % rep
        assert torch.equal(out_g.view(torch.int32), out_e.view(torch.int32)), \
            "replay %d: output differs from the eager pass" % rep
        if rep == 0:
            ref, ref_idx, _, _ = oracle.Layer(case).forward()
            assert (idx_g.cpu().numpy() == ref_idx).all(1).mean() >= 0.95
            assert_normwise(out_g.cpu().numpy(), ref, tol_of(case), "graph replay vs oracle")


PRENORM = [
    ("qwen35moe_decode", 8, dict(E=32, H=256, F=128, Fs=128, k=4)),   # norm inside the router product
    ("qwen35moe_decode", 300, dict(E=16, H=256, F=192, Fs=128, k=4)),  # RMSNorm launch + MFMA path
]


@pytest.mark.parametrize("name,T,over", PRENORM, ids=[_ids(p) for p in PRENORM])
def test_prenorm_graph_replay(name, T, over):
    """moe_forward_prenorm captured once, replayed on new residual rows, each
    replay bit-equal to an eager pass."""
    log("prenorm graph replay: %s T=%d %s" % (name, T, over))
    case = synth.add_block_inputs(synth.make_case(name, T=T, **over))
    cfg = config_of(case)
    w = device_weights(case)
    g_w = to_torch(case.t["norm_w"])
    rs = [case.t["resid"]] + [synth.add_block_inputs(synth.make_case(name, T=T, only={"x"}, **over),
                                                     seed=synth.BASE_SEED + i).t["resid"] for i in (1, 2, 3)]
    r_static = to_torch(rs[0])
    out_g = torch.empty((T, case.H), dtype=torch.float32, device="cuda")
    ws_g = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    out_e, ws_e = torch.empty_like(out_g), torch.empty_like(ws_g)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.moe_forward_prenorm(cfg, w, g_w, case.norm_eps, r_static, T, out_g, ws_g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_forward_prenorm(cfg, w, g_w, case.norm_eps, r_static, T, out_g, ws_g)
    torch.cuda.synchronize()
    for rep, r in enumerate(rs):
        r_static.copy_(to_torch(r))
        out_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        moe.moe_forward_prenorm(cfg, w, g_w, case.norm_eps, to_torch(r), T, out_e, ws_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int32), out_e.view(torch.int32)), \
            "replay %d: output differs from the eager pass" % rep


@pytest.mark.parametrize("name,T,over", CASES[:2], ids=[_ids(p) for p in CASES[:2]])
def test_chain_of_passes_in_one_graph(name, T, over):
    """Four passes captured one after the other in a single graph (each its
    own input and output, one shared workspace, as consecutive layers would
    share it), replayed on new inputs with eager passes between the replays:
    every pass of every replay bit-equal to an eager pass on its input."""
    log("graph chain: %s T=%d %s" % (name, T, over))
    case = synth.make_case(name, T=T, **over)
    cfg = config_of(case)
    w = device_weights(case)
    L = 4

    def draw(r):
        return [synth.make_case(name, T=T, seed=synth.BASE_SEED + 10 * r + i, only={"x"}, **over).t["x"]
                for i in range(L)]

    x_static = [to_torch(x) for x in draw(0)]
    outs = [torch.empty((T, case.H), dtype=torch.float32, device="cuda") for _ in range(L)]
    ws = torch.empty(moe.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    out_e = torch.empty_like(outs[0])
    ws_e = torch.empty_like(ws)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(L):
            moe.moe_forward(cfg, w, x_static[i], T, outs[i], ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(L):
            moe.moe_forward(cfg, w, x_static[i], T, outs[i], ws)
    torch.cuda.synchronize()
    for rep in range(3):
        xs = draw(rep)
        for i in range(L):
            x_static[i].copy_(to_torch(xs[i]))
            outs[i].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i in range(L):
            moe.moe_forward(cfg, w, to_torch(xs[i]), T, out_e, ws_e)
            torch.cuda.synchronize()
            assert torch.equal(outs[i].view(torch.int32), out_e.view(torch.int32)), \
                "replay %d, pass %d: output differs from the eager pass" % (rep, i)

"""Benchmark of the MoE FFN layer on one MI355X.

Default workload: the qwen35moe-shaped decode layer (T=8 tokens, H=2048,
256 experts, top-8, expert FF 512, shared expert FF 512, bf16 weights and
activations, fp32 router).  A step is one whole-layer pass (moe_forward:
router product, gating, permutation, expert gate/up + SwiGLU, down +
weighted combine + shared expert) over one batch of synthetic tokens, with
inputs resident in HBM.  Steps rotate over four seeded token batches (each
routes to its own set of experts) and over four identical weight copies at
different addresses, so every step streams its experts cold from HBM (the
256 MB last-level cache never holds the previous step's experts), as
consecutive layers of a model would.

The same JSON line also reports the prefill-sized layer (same weights,
T=4096 tokens, router logits drawn so expert load is Zipf(1.0)-skewed), the
gpt-oss-20b-shaped layers (bf16 T=2048; MXFP4 experts at T=16 and T=2048;
the MXFP8-input mode of the MXFP4 layer), each against its roofline, the
roofline of the decode layer's dominant kernel and the CPU oracle's
throughput (one thread and all threads).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-prefill] [--no-gptoss]
       python bench.py --pmc-summary FETCH_DIR WRITE_DIR   (HBM traffic from two rocprofv3 --pmc runs)

HBM traffic of the dominant kernel comes from two rocprofv3 counter runs of
this script with --copy-calib-mib (FETCH_SIZE, then WRITE_SIZE); each counter
is scaled by what it reads for a plain device copy of known size in the same
run.  The summary written by --pmc-summary is kept next to the kernel
profiles and carries a hash of the kernel's source: the JSON line reports the
traffic only while that hash matches the current source.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec + %HBM-roofline (T=8 decode) and %MFMA-peak (T=4096)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
N_BATCHES = 4  # seeded token batches the decode steps rotate over
GATEUP_KERNEL = "k_gateup_gemv"
COPY_KERNEL = "__amd_rocclr_copyBuffer"
KERNEL_SOURCES = ("sparse_moe_ffn_router_amd/csrc/ffn_gemv.hip", "sparse_moe_ffn_router_amd/csrc/moe_internal.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_gateup_gemv_qwen35moe_decode_T8_hbm_traffic.txt")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated per step")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-prefill", action="store_true", help="skip the T=4096 measurement")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the pre-norm block measurement (its residual rows route to other experts, so "
                         "counter runs of the decode gate/up kernel leave it out)")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--cpu-run-seconds", type=float, default=1.5,
                    help="length of each of the 5 timed oracle runs per form")
    ap.add_argument("--no-gptoss", action="store_true",
                    help="skip the gpt-oss-20b-shaped layers (bf16 T=2048, MXFP4 T=16 and T=2048)")
    ap.add_argument("--batches", type=int, default=N_BATCHES, help="seeded token batches the decode steps rotate over")
    ap.add_argument("--only", choices=("decode", "prefill", "gptoss"),
                    help="measure one workload only (counter runs); no JSON line")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="after the measurements, copy a buffer of this many MiB 5 times (counter calibration)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc output folders and exit")
    ap.add_argument("--pmc-kernels", default=GATEUP_KERNEL,
                    help="semicolon-separated kernel name fragments the summary reports (first: the traffic line)")
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


class Layer:
    """Device-resident layer: weight copies, one batch of tokens, outputs."""

    def __init__(self, case, copies, T=None, logits=None, x=None, xs=None):
        import torch
        from tests._gpu import config_of, device_weights, to_torch
        import sparse_moe_ffn_router_amd as moe
        self.moe = moe
        self.case = case
        self.T = case.T if T is None else T
        self.cfg = config_of(case)
        base = device_weights(case)
        if logits is not None:
            base = {k: v for k, v in base.items() if k not in ("router_w", "router_b")}
        self.weights = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(copies - 1)]
        # token batches; step s runs batch s % len(xs) on weight copy s % copies
        self.xs = [to_torch(b) for b in xs] if xs else [to_torch(case.t["x"] if x is None else x)]
        self.x = self.xs[0]
        self.logits = to_torch(logits) if logits is not None else \
            torch.empty((self.T, case.E), dtype=torch.float32, device="cuda")
        self.out = torch.empty((self.T, case.H), dtype=torch.float32, device="cuda")
        self.idx = torch.empty((self.T, case.k), dtype=torch.int32, device="cuda")
        self.wt = torch.empty((self.T, case.k), dtype=torch.float32, device="cuda")
        self.sg = torch.empty(self.T, dtype=torch.float32, device="cuda")
        self.ws = torch.empty(moe.moe_workspace_bytes(self.cfg, self.T), dtype=torch.uint8, device="cuda")
        n_rows = self.T * case.k + (self.T if case.has_shared else 0)
        self.offsets = torch.empty(case.E + 2, dtype=torch.int32, device="cuda")
        self.sorted = torch.empty(n_rows, dtype=torch.int32, device="cuda")
        self.pos = torch.empty(n_rows, dtype=torch.int32, device="cuda")
        self.h = torch.empty(self.T * case.k * case.F + (self.T * case.Fs if case.has_shared else 0),
                             dtype=torch.bfloat16, device="cuda")

    def forward(self, step):
        self.moe.moe_forward(self.cfg, self.weights[step % len(self.weights)], self.xs[step % len(self.xs)], self.T,
                             self.out, self.ws, logits=self.logits, topk_idx=self.idx, topk_w=self.wt, sgate=self.sg)

    def forward_batch(self, b):
        """Steps over batch b alone (weight copies still rotate)."""
        return lambda step: self.moe.moe_forward(self.cfg, self.weights[step % len(self.weights)], self.xs[b],
                                                 self.T, self.out, self.ws, logits=self.logits, topk_idx=self.idx,
                                                 topk_w=self.wt, sgate=self.sg)

    def block(self, step):
        """The layer inside its pre-norm block (RMSNorm in front, residual add
        behind) on residual rows of the same batch size."""
        if not hasattr(self, "resid"):
            import synth
            from tests._gpu import to_torch
            synth.add_block_inputs(self.case)
            self.resid = to_torch(self.case.t["resid"])
            self.norm_w = to_torch(self.case.t["norm_w"])
            self.xn = torch_empty_like(self.x)
        self.moe.moe_forward_prenorm(self.cfg, self.weights[step % len(self.weights)], self.norm_w,
                                     self.case.norm_eps, self.resid, self.T, self.out, self.ws, xn=self.xn,
                                     logits=self.logits, topk_idx=self.idx, topk_w=self.wt, sgate=self.sg)

    def forward_on_xn(self, step):
        """The plain layer on the normalised rows the block produced (the
        same routing, so the block's own cost shows)."""
        self.moe.moe_forward(self.cfg, self.weights[step % len(self.weights)], self.xn, self.T, self.out, self.ws,
                             logits=self.logits, topk_idx=self.idx, topk_w=self.wt, sgate=self.sg)

    def ops(self, step, ev_ffn=None):
        """The same kernels through the four step entry points; optional
        events bracket the expert gate/up launch."""
        m, w, x = self.moe, self.weights[step % len(self.weights)], self.xs[step % len(self.xs)]
        m.moe_route(self.cfg, w, x, self.logits, self.idx, self.wt, self.sg, self.T, self.ws)
        m.moe_permute(self.cfg, self.idx, self.T, self.offsets, self.sorted, self.pos, self.ws)
        if ev_ffn:
            ev_ffn[0].record()
        m.moe_expert_ffn(self.cfg, w, x, self.offsets, self.sorted, self.T, self.h)
        if ev_ffn:
            ev_ffn[1].record()
        m.moe_combine(self.cfg, w, self.h, self.offsets, self.sorted, self.wt, self.sg, self.T, self.out, self.ws)


def torch_empty_like(t):
    import torch
    return torch.empty_like(t)


def time_loop(fn, steps, warmup):
    import torch
    for s in range(warmup):
        fn(s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for s in range(steps):
        fn(warmup + s)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def graph_replay_ms(layer, steps, warmup):
    """moe_forward captured in one HIP graph per (batch, weight copy) pair of
    the rotation, replayed in the same rotation as the eager loop."""
    import math
    import torch
    n = len(layer.weights) * len(layer.xs) // math.gcd(len(layer.weights), len(layer.xs))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in range(n):
            layer.forward(c)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graphs = []
    for c in range(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer.forward(c)
        graphs.append(g)
    torch.cuda.synchronize()
    ms, _ = time_loop(lambda st: graphs[st % len(graphs)].replay(), steps, warmup)
    return ms


def graph_chain_ms(layer, steps, warmup):
    """The passes of the whole (batch, weight copy) rotation captured one
    after the other in a single HIP graph -- as a model's graph holds its
    consecutive layers -- replayed; time per pass."""
    import math
    import torch
    n = len(layer.weights) * len(layer.xs) // math.gcd(len(layer.weights), len(layer.xs))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in range(n):
            layer.forward(c)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in range(n):
            layer.forward(c)
    torch.cuda.synchronize()
    ms, _ = time_loop(lambda st: g.replay(), max(steps // n, 10), max(warmup // n, 2))
    return ms / n, n


def active_experts(idx_np, E):
    import numpy as np
    return int(np.unique(idx_np.reshape(-1)).size)


def gateup_bytes(case, n_active, T):
    """Algorithmic bytes of one expert gate/up launch: every active routed
    expert's gate and up rows once (2*F*H bf16 = 4 MiB each for this shape),
    the shared expert's, the tokens read and h written."""
    w = n_active * 2 * case.F * case.H * 2
    if case.has_shared:
        w += 2 * case.Fs * case.H * 2
    x = T * case.H * 2
    h = (T * case.k * case.F + (T * case.Fs if case.has_shared else 0)) * 2
    return w + x + h


def layer_bytes(case, n_active, T):
    """Algorithmic bytes of the whole layer: active experts' weights, router,
    shared expert, tokens in, fp32 out."""
    per_expert = 3 * case.F * case.H * 2
    b = n_active * per_expert + case.E * case.H * 2 + T * case.H * 2 + T * case.H * 4
    if case.has_shared:
        b += 3 * case.Fs * case.H * 2 + case.H * 2
    return b


def gptoss_layer_bytes(case, n_active, T):
    """Algorithmic bytes of a gpt-oss-shaped layer: every active expert's
    gate_up and down weights once (bf16: 2 bytes per weight; MXFP4: half a
    byte of code plus one E8M0 byte per 32 weights) and its bf16 biases, the
    router and its bias, tokens in (bf16) and out (fp32)."""
    per_w = 2.0 if case.w_dtype == "bf16" else 0.5 + 1.0 / 32.0
    per_expert = (2 * case.F * case.H + case.H * case.F) * per_w + (2 * case.F + case.H) * 2
    b = n_active * per_expert + case.E * case.H * 2 + case.E * 2 + T * case.H * 2 + T * case.H * 4
    if case.has_shared:
        b += 3 * case.Fs * case.H * 2 + case.H * 2
    return b


def layer_flops(case, T):
    f = 2 * T * case.k * 3 * case.F * case.H + 2 * T * case.H * case.E
    if case.has_shared:
        f += 2 * T * 3 * case.Fs * case.H + 2 * T * case.H
    return f


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _pmc_means(folder, counter, kernels):
    """Mean counter value per dispatch (KiB for FETCH_SIZE / WRITE_SIZE) of
    each kernel (name fragment) and of the calibration copies, from a
    rocprofv3 --pmc csv folder.  The calibration copies are the copy
    dispatches issued after every measured kernel's last dispatch."""
    rows = []
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += [r for r in csv.DictReader(fh) if r["Counter_Name"] == counter]
    mean = lambda rs: (sum(float(r["Counter_Value"]) for r in rs) / len(rs), len(rs)) if rs else (0.0, 0)
    out, last = {}, 0
    for k in kernels:
        ks = [r for r in rows if k in r["Kernel_Name"]]
        out[k] = mean(ks)
        if ks:
            last = max(last, max(int(r["Dispatch_Id"]) for r in ks))
    out[COPY_KERNEL] = mean([r for r in rows if r["Kernel_Name"] == COPY_KERNEL and int(r["Dispatch_Id"]) > last])
    return out


def pmc_summary(fetch_dir, write_dir, copy_mib, kernels):
    """Text summary: each kernel's FETCH_SIZE and WRITE_SIZE per launch, each
    scaled by copy bytes / the copy kernel's counter.  The first kernel's
    total is the traffic line the JSON output reads back."""
    copy_bytes = copy_mib * 2 ** 20
    out, total = [], {k: 0.0 for k in kernels}
    for counter, folder in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        m = _pmc_means(folder, counter, kernels)
        ck, cn = m[COPY_KERNEL]
        factor = copy_bytes / (ck * 1024.0)
        out.append("%s: copy of %d bytes counts %.1f KiB/dispatch (%d dispatches) -> factor %.4f" %
                   (counter, copy_bytes, ck, cn, factor))
        for k in kernels:
            gk, gn = m[k]
            b = gk * 1024.0 * factor
            total[k] += b
            out.append("%s: %s %.1f KiB/dispatch (%d dispatches) -> %.0f bytes per launch" % (counter, k, gk, gn, b))
    for k in kernels[1:]:
        out.append("traffic %s = %.0f bytes per launch" % (k, total[k]))
    out += ["traffic_bytes_per_launch = %.0f" % total[kernels[0]], "source_sha256 = %s" % kernel_source_hash()]
    return "\n".join(out)


def recorded_traffic():
    """HBM bytes per launch of the gate/up kernel from the committed counter
    summary, or None when it is missing or the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(l.split(" = ", 1) for l in f.read().splitlines() if " = " in l)
        if kv.get("source_sha256", "").strip() != kernel_source_hash():
            return None
        return int(float(kv["traffic_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(case, run_seconds):
    """The oracle (plain C, double accumulation, OpenMP over tokens) on the
    decode batch: 5 timed runs of a fixed number of whole-batch passes (sized
    to about run_seconds each), median, with one thread and with all the
    threads the process may use."""
    import statistics
    import oracle
    L = oracle.Layer(case)
    avail = len(os.sched_getaffinity(0))
    forms = {}
    for name, threads in (("single_thread", 1), ("openmp", avail)):
        oracle.set_threads(threads)
        t0 = time.perf_counter()
        L.forward()
        reps = max(1, int(run_seconds / max(time.perf_counter() - t0, 1e-6)))
        runs = []
        for _ in range(5):
            t0 = time.perf_counter()
            for _ in range(reps):
                L.forward()
            runs.append(time.perf_counter() - t0)
        med = statistics.median(runs)
        forms[name] = {"value": round(reps * case.T / med, 3), "unit": "tokens/s",
                       "cores": min(threads, case.T), "threads": threads,
                       "runs_s": [round(r, 3) for r in runs], "passes_per_run": reps}
    oracle.set_threads(avail)
    omp = forms["openmp"]
    return {"value": omp["value"], "unit": "tokens/s", "cores": omp["cores"], "kind": "oracle",
            "sample": "median of 5 runs of %d passes over the whole T=%d decode batch, OpenMP over tokens "
                      "(%d threads available, at most %d busy: one per token)" % (omp["passes_per_run"], case.T,
                                                                                  avail, case.T),
            "nproc": avail, "single_thread": forms["single_thread"], "openmp": forms["openmp"]}


def main():
    a = parse()
    if a.pmc_summary:
        print(pmc_summary(a.pmc_summary[0], a.pmc_summary[1], a.copy_calib_mib or 1024, a.pmc_kernels.split(";")))
        return
    if a.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (requested --gpus %d)" % a.gpus,
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import synth

    torch.cuda.set_device(0)
    t0 = time.perf_counter()
    dec = synth.make_case("qwen35moe_decode", T=8)
    # seeded token batches of the same layer: batch 0 is the case's own x
    xs = [dec.t["x"]] + [synth.normal("x", (dec.T, dec.H), 1.0, "bf16", synth.BASE_SEED + b) for b in range(1, a.batches)]
    log("decode case generated in %.1f s" % (time.perf_counter() - t0))
    result = {}
    if a.only in (None, "decode"):
        layer = Layer(dec, a.copies, xs=xs)
        per_batch = []
        for b in range(len(xs)):
            b_ms, _ = time_loop(layer.forward_batch(b), max(a.steps // 2, 20), a.warmup)
            per_batch.append({"batch": b, "ms_per_step": round(b_ms, 5), "tokens_per_s": round(dec.T / (b_ms * 1e-3), 1),
                              "active_experts": active_experts(layer.idx.cpu().numpy(), dec.E)})
        ms, wall = time_loop(layer.forward, a.steps, a.warmup)
        actives = [p_["active_experts"] for p_ in per_batch]
        tok_s = dec.T / (ms * 1e-3)
        log("decode: %.4f ms/step, %.0f tokens/s over %d batches (active experts %s)" % (ms, tok_s, len(xs), actives))
        g_ms = graph_replay_ms(layer, a.steps, a.warmup)
        log("decode, HIP graph replay: %.4f ms/step" % g_ms)
        gc_ms, gc_n = graph_chain_ms(layer, a.steps, a.warmup)
        log("decode, %d passes in one HIP graph: %.4f ms/pass" % (gc_n, gc_ms))
        block = None
        if not a.no_block:
            b_ms, _ = time_loop(layer.block, a.steps, a.warmup)
            b_active = active_experts(layer.idx.cpu().numpy(), dec.E)
            bx_ms, _ = time_loop(layer.forward_on_xn, a.steps, a.warmup)
            log("decode, pre-norm block (RMSNorm + layer + residual): %.4f ms/step; the layer alone on the same "
                "normalised rows %.4f ms (%d active experts)" % (b_ms, bx_ms, b_active))
            block = {"ms_per_step": round(b_ms, 5), "tokens_per_s": round(dec.T / (b_ms * 1e-3), 1),
                     "layer_on_same_rows_ms": round(bx_ms, 5), "over_layer_ms": round(b_ms - bx_ms, 5),
                     "active_experts": b_active,
                     "note": "moe_forward_prenorm on residual rows (RMSNorm in the router-product kernel, "
                             "residual add in the combine) against moe_forward on the rows it normalised"}

        # dominant kernel (expert gate/up), timed with events on the launch stream
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
        for s in range(a.warmup):
            layer.ops(s)
        torch.cuda.synchronize()
        for s in range(a.steps):
            layer.ops(a.warmup + s, evs[s])
        torch.cuda.synchronize()
        k_times = [e0.elapsed_time(e1) for e0, e1 in evs]
        k_ms = float(np.mean(k_times))
        k_bytes = [gateup_bytes(dec, actives[(a.warmup + s) % len(xs)], dec.T) for s in range(a.steps)]
        gb = float(np.mean(k_bytes))
        achieved = sum(k_bytes) / (sum(k_times) * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": "k_gateup_gemv (expert gate/up + SwiGLU)", "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": recorded_traffic(),
                    "kernel_ms": round(k_ms, 5), "algorithmic_bytes": round(gb)}
        lb = float(np.mean([layer_bytes(dec, n, dec.T) for n in actives]))
        layer_gbs = lb / (ms * 1e-3) / 1e9

        result = {
            "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
            "warmup": a.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "qwen35moe-shaped decode MoE layer", "tokens": dec.T, "hidden": dec.H,
                       "n_expert": dec.E, "top_k": dec.k, "expert_ff": dec.F, "shared_ff": dec.Fs,
                       "token_batches_rotated": len(xs), "active_experts_per_batch": actives,
                       "weight_copies_rotated": a.copies,
                       "layer_algorithmic_bytes": round(lb), "layer_GBps": round(layer_gbs, 1),
                       "layer_frac_hbm": round(layer_gbs / HBM_PEAK_GBS, 4), "wall_s": round(wall, 3),
                       "per_batch": per_batch},
            "graph_replay": {"ms_per_step": round(g_ms, 5), "tokens_per_s": round(dec.T / (g_ms * 1e-3), 1),
                             "note": "the same moe_forward passes captured once per (batch, weight copy) in HIP graphs"},
            "graph_chain": {"ms_per_step": round(gc_ms, 5), "tokens_per_s": round(dec.T / (gc_ms * 1e-3), 1),
                            "passes_per_graph": gc_n,
                            "note": "the rotation's passes captured one after the other in a single HIP graph, as "
                                    "a model's graph holds consecutive layers; time per pass"},
            "prenorm_block": block,
            "roofline": roofline,
        }
        del layer
        torch.cuda.empty_cache()

    if not a.no_prefill and a.only in (None, "prefill"):
        T = 4096
        pre = synth.make_case("qwen35moe_prefill_zipf", T=T, only={"x", "logits"})
        pre.t.update({k: v for k, v in dec.t.items() if k != "x"})
        pl = Layer(pre, a.copies, logits=pre.t["logits"])
        p_ms, _ = time_loop(pl.forward, a.prefill_steps, 3)
        # the drawn logits skip the router product; time it at the same shape
        # (this batch's tokens, the decode layer's router) as the routing
        # step with the product minus the routing step on the drawn logits
        # (the gating, which the layer above already ran), and add that
        rt = Layer(dec, 1, T=T, x=pre.t["x"])
        route_ms, _ = time_loop(lambda s: rt.moe.moe_route(rt.cfg, rt.weights[0], rt.x, rt.logits, rt.idx, rt.wt,
                                                            rt.sg, T, rt.ws), a.prefill_steps, 3)
        gate_ms, _ = time_loop(lambda s: pl.moe.moe_route(pl.cfg, pl.weights[0], pl.x, pl.logits, pl.idx, pl.wt,
                                                           pl.sg, T, pl.ws), a.prefill_steps, 3)
        r_ms = max(route_ms - gate_ms, 0.0)
        tot = p_ms + r_ms
        fl = layer_flops(pre, T)
        tf = fl / (tot * 1e-3) / 1e12
        pb = layer_bytes(pre, pre.E, T)
        attainable = min(BF16_PEAK_TFLOPS, fl / pb * HBM_PEAK_GBS / 1e3)
        result["prefill"] = {
            "workload": "qwen35moe-shaped prefill MoE layer, Zipf(1.0) expert load", "tokens": T,
            "ms_per_step": round(tot, 4), "layer_ms_drawn_logits": round(p_ms, 4), "router_ms": round(r_ms, 4),
            "route_ms_with_router": round(route_ms, 4), "route_ms_drawn_logits": round(gate_ms, 4),
            "tokens_per_s": round(T / (tot * 1e-3), 1), "TFLOPs": round(tf, 2),
            "frac_bf16_mfma_peak": round(tf / BF16_PEAK_TFLOPS, 4), "algorithmic_flops": fl,
            "algorithmic_bytes": pb, "frac_hbm": round(pb / (tot * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "attainable_TFLOPs": round(attainable, 1), "frac_attainable": round(tf / attainable, 4)}
        log("prefill: %.3f ms (+router %.3f ms), %.1f TFLOP/s" % (p_ms, r_ms, tf))
        del pl, rt
        torch.cuda.empty_cache()

    if not a.no_gptoss and a.only in (None, "gptoss"):
        result["gptoss"] = {}
        for name, T, aq in (("gptoss20b_bf16", 2048, "none"), ("gptoss20b_mxfp4", 16, "none"),
                            ("gptoss20b_mxfp4", 2048, "none"), ("gptoss20b_mxfp4", 16, "mxfp8"),
                            ("gptoss20b_mxfp4", 2048, "mxfp8")):
            c = synth.make_case(name, T=T)
            c.act_quant = aq
            few = T <= 64
            gxs = [c.t["x"]] + ([synth.normal("x", (T, c.H), 1.0, "bf16", synth.BASE_SEED + b)
                                 for b in range(1, a.batches)] if few else [])
            gl = Layer(c, a.copies if few else 2, xs=gxs)
            n_act = []
            for b in range(len(gxs)):
                gl.forward_batch(b)(0)
                torch.cuda.synchronize()
                n_act.append(active_experts(gl.idx.cpu().numpy(), c.E))
            g_ms, _ = time_loop(gl.forward, a.steps if few else a.prefill_steps, 3 if not few else a.warmup)
            byt = float(np.mean([gptoss_layer_bytes(c, n, T) for n in n_act]))
            fl = layer_flops(c, T)
            tf = fl / (g_ms * 1e-3) / 1e12
            key = "%s_T%d%s" % (name, T, "_mxfp8_act" if aq == "mxfp8" else "")
            rec = {"ms": round(g_ms, 4), "tokens_per_s": round(T / (g_ms * 1e-3), 1), "TFLOPs": round(tf, 2),
                   "algorithmic_bytes": round(byt), "frac_hbm": round(byt / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                   "active_experts": n_act if few else n_act[0]}
            if not few:
                peak = FP8_PEAK_TFLOPS if aq == "mxfp8" else BF16_PEAK_TFLOPS
                rec["bound"] = "fp8 mfma" if aq == "mxfp8" else "bf16 mfma"
                rec["frac_mfma_peak"] = round(tf / peak, 4)
                rec["attainable_TFLOPs"] = round(min(peak, fl / byt * HBM_PEAK_GBS / 1e3), 1)
                rec["frac_attainable"] = round(tf / rec["attainable_TFLOPs"], 4)
            else:
                rec["bound"] = "hbm"
                rec["token_batches_rotated"] = len(gxs)
            result["gptoss"][key] = rec
            log("%s: %s" % (key, rec))
            del gl, c
            torch.cuda.empty_cache()

    if a.copy_calib_mib:
        src = torch.empty(a.copy_calib_mib * 2 ** 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if a.only:
        return
    if not a.no_cpu:
        result["cpu_baseline"] = cpu_baseline(dec, a.cpu_run_seconds)
        log("cpu oracle: %s" % result["cpu_baseline"])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

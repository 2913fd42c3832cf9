"""Shared parity helpers for the GPU tests (tolerances and comparisons).

Output tolerances are normwise, max|gpu - ref| <= tol * max|ref|: 1e-4 for
fp32 layers, 2e-2 for bf16 weights, 3e-2 for MXFP4 weights.  Routing weights
and the shared gate: <= 1e-5 relative per element (softmax / sigmoid in
fp32, "qwen35moe CPU-reference golden vectors", Kernel 4 tolerance)."""
import sys

import numpy as np

import synth

TOL = {"f32": 1e-4, "bf16": 2e-2, "mxfp4": 3e-2}


def tol_of(case):
    return TOL[case.w_dtype]


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


_WEIGHTS = {}


def cached_case(name, T, only=None):
    """make_case(name, T), with the weights of each named case generated once
    per process (they do not depend on T; tokens and drawn logits do)."""
    if only is not None or name == "tiny_fp32":
        return synth.make_case(name, T=T, only=None if only is None else set(only))
    if name not in _WEIGHTS:
        c = synth.make_case(name, T=T)
        _WEIGHTS[name] = {k: v for k, v in c.t.items() if k not in ("x", "logits")}
        return c
    c = synth.make_case(name, T=T, only={"x", "logits"})
    c.t.update(_WEIGHTS[name])
    return c


def normwise(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    return err, scale


def assert_normwise(got, ref, tol, what=""):
    err, scale = normwise(got, ref)
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    assert err <= tol * scale, "%s: max|err| %.3e > %.1e * max|ref| %.3e" % (what, err, tol, scale)
    return err / scale if scale else 0.0


def assert_rel(got, ref, rtol, atol=0.0, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    bad = np.abs(got - ref) > rtol * np.abs(ref) + atol
    assert not bad.any(), "%s: %d elements beyond %.1e relative, worst %s vs %s" % (
        what, int(bad.sum()), rtol, got[bad][:4], ref[bad][:4])

"""Shared parity helpers for the GPU tests (tolerances and comparisons).

Output tolerances are normwise, max|gpu - ref| <= tol * max|ref|: 1e-4 for
fp32 layers, 2e-2 for bf16 weights, 3e-2 for MXFP4 weights.  Routing weights
and the shared gate: <= 1e-5 relative per element (softmax / sigmoid in
fp32, "qwen35moe CPU-reference golden vectors", Kernel 4 tolerance)."""
import os
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
    per process (they do not depend on T; tokens and drawn logits do).  With
    MOE_CASE_CACHE set to a directory, cases are also kept there as vector
    files (synth.vecfile) and read back by later runs."""
    cache_dir = os.environ.get("MOE_CASE_CACHE")
    if cache_dir and only is None:
        return synth.vecfile.cached_case(cache_dir, name, T)
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


def logit_bound(case, tokens, x=None):
    """fp32 dot-product error bound of the GPU's router logits for the given
    tokens, per (token, expert): H * 2^-24 * sum |x||w| (Higham), plus one
    fp32 step.  Zero when the logits are given (drawn) rather than computed."""
    if case.drawn_logits:
        return np.zeros((len(tokens), case.E))
    xs = case.t["x"] if x is None else x
    f64 = lambda a, dt: synth.bf16_to_f32(a).astype(np.float64) if dt == "bf16" else np.asarray(a, np.float64)
    xa = np.abs(f64(xs[tokens], case.x_dtype))
    wa = np.abs(f64(case.t["router_w"], case.router_dtype))
    return case.H * 2.0 ** -24 * (xa @ wa.T) + 2.0 ** -23


def check_layer_output(case, tokens, g_idx, g_out, r_out, r_idx, ref_logits, redo, tol, what="layer output",
                       exact_routing=False, x=None):
    """Routing and output of a whole-layer pass against the oracle.

    g_idx, g_out: the GPU's picks [T][k] and output rows (all tokens);
    r_out, r_idx: the oracle's, on its own routing (rows `tokens` valid);
    ref_logits: the oracle's logits of the sampled tokens;
    redo(idx, tokens): the oracle's output rows when it takes the given picks.

    With exact_routing (the same logits on both sides) every sampled token
    must route identically.  Otherwise a token may route differently only if
    the oracle's logits leave a gap inside the rounding bound of the GPU's;
    such a token's output is then compared with the oracle's output on the
    GPU's own picks, at the same tolerance.  Returns max|err|/max|ref|."""
    g_i, r_i = g_idx[tokens], r_idx[tokens]
    same = (g_i == r_i).all(1)
    ref = np.array(r_out[tokens], np.float64)
    if exact_routing:
        assert same.all(), "%d of %d tokens routed differently on identical logits" % ((~same).sum(), len(tokens))
    elif not same.all():
        bnd = logit_bound(case, tokens, x)
        for i in np.nonzero(~same)[0]:
            kth = np.sort(ref_logits[i])[::-1][case.k - 1]
            sel = set(g_i[i].tolist())
            assert len(sel) == case.k and all(0 <= e < case.E for e in sel), "token %d: invalid picks" % i
            for e in range(case.E):
                if e in sel:
                    assert ref_logits[i, e] >= kth - 2 * bnd[i].max(), "token %d: GPU picked a clearly losing expert" % i
                else:
                    assert ref_logits[i, e] <= kth + 2 * bnd[i].max(), "token %d: GPU dropped a clear winner" % i
        diff = np.asarray(tokens)[~same]
        ref[~same] = np.asarray(redo(g_idx, diff), np.float64)[diff]
        log("  %d of %d sampled tokens routed differently inside the rounding bound; compared on the GPU's picks"
            % ((~same).sum(), len(tokens)))
    return assert_normwise(g_out[tokens], ref, tol, what)

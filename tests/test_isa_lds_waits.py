"""Every LDS read of the HIP kernels completes before its registers are used.

The grouped GEMMs read their MFMA operands from LDS through inline asm (so
the compiler adds no waits for the buffer->LDS loads in flight) and wait
for them with their own ``s_waitcnt lgkmcnt``.  The compiler does not see
those reads as loads: if register allocation ever copied or reused a
destination register between such a read and its wait, the copy would
take stale data, silently.  This test compiles each kernel source to
gfx950 assembly and follows every control-flow path from every LDS read
until an ``s_waitcnt lgkmcnt(n)`` provably covers it (LDS operations
complete in order, so n no larger than the LGKM operations issued after
the read); any other instruction touching the read's destination
registers on the way is a failure.  A later LDS read writing the same
registers is allowed (in-order completion).  CPU only: needs hipcc, no
GPU.
"""
import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_moe_ffn_router_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]

_LGKM_WRITERS = ("ds_read", "ds_bpermute", "ds_permute", "ds_swizzle")


def _vregs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _kernels(asm):
    """[(name, [(line, text)], {label: index})] of the functions in an assembly listing."""
    out, cur = [], None
    for ln, raw in enumerate(asm.split("\n"), 1):
        if re.match(r"^_Z\S*:|^[A-Za-z_]\w*:\s*; @", raw):
            cur = (raw.split(":")[0], [], {})
            out.append(cur)
            continue
        if cur is None:
            continue
        if raw.startswith(".Lfunc_end"):
            cur = None
            continue
        m = re.match(r"^(\.LBB\d+_\d+):", raw)
        if m:
            cur[2][m.group(1)] = len(cur[1])
            continue
        t = raw.split(";")[0].strip()
        if t and not t.startswith("."):
            cur[1].append((ln, t))
    return out


def pending_uses(asm):
    """(read line, use line, use text) for every use of a pending LDS read's destination."""
    found = []
    for _, ins, lab in _kernels(asm):
        for i, (ln, t) in enumerate(ins):
            op = t.split()[0]
            if not op.startswith(_LGKM_WRITERS):
                continue
            dst = _vregs(t[len(op):].split(",")[0].strip())
            seen, stack = set(), [(i + 1, 0)]
            while stack:
                j, after = stack.pop()
                if j >= len(ins) or (j, min(after, 64)) in seen:
                    continue
                seen.add((j, min(after, 64)))
                ln2, t2 = ins[j]
                op2 = t2.split()[0]
                if op2 == "s_waitcnt":
                    m = re.search(r"lgkmcnt\((\d+)\)", t2)
                    if not (m and after >= int(m.group(1))):
                        stack.append((j + 1, after))
                    continue
                if op2 in ("s_endpgm", "s_setpc_b64"):
                    continue
                if op2 == "s_branch":
                    stack.append((lab[t2.split()[1]], after))
                    continue
                if op2.startswith("s_cbranch"):
                    stack.append((lab[t2.split()[1]], after))
                    stack.append((j + 1, after))
                    continue
                used = set()
                for tok in t2[len(op2):].split(","):
                    used |= _vregs(tok.strip())
                if used & dst and not op2.startswith(_LGKM_WRITERS):
                    found.append((ln, ln2, t2))
                if op2.startswith("ds_") or op2.startswith("s_load") or op2.startswith("s_buffer_load"):
                    after += 1
                stack.append((j + 1, after))
    return sorted(set(found))


# --- the checker itself, on hand-written listings ---------------------------------------------

_OK = """_Z1kv:
	ds_read_b128 v[4:7], v1
	ds_read_b128 v[8:11], v2
	s_waitcnt lgkmcnt(1)
	v_mov_b32_e32 v20, v4
	s_waitcnt lgkmcnt(0)
	v_mov_b32_e32 v21, v8
	s_endpgm
.Lfunc_end0:
"""
_BAD = """_Z1kv:
	ds_read_b128 v[4:7], v1
	ds_read_b128 v[8:11], v2
	s_waitcnt lgkmcnt(1)
	v_mov_b32_e32 v21, v8
	s_endpgm
.Lfunc_end0:
"""
_BACKEDGE = """_Z1kv:
.LBB0_1:
	v_mov_b32_e32 v30, v4
	ds_read_b128 v[4:7], v1
	s_cbranch_scc1 .LBB0_1
	s_waitcnt lgkmcnt(0)
	s_endpgm
.Lfunc_end0:
"""
_WAW_LDS = """_Z1kv:
	ds_read_b128 v[4:7], v1
	ds_read_b128 v[4:7], v2
	s_waitcnt lgkmcnt(0)
	v_mov_b32_e32 v20, v4
	s_endpgm
.Lfunc_end0:
"""


def test_checker_flags_a_use_before_the_covering_wait():
    assert pending_uses(_OK) == []
    bad = pending_uses(_BAD)
    assert [b[1] for b in bad] == [5] and "v8" in bad[0][2]


def test_checker_follows_back_edges_and_allows_in_order_lds_overwrites():
    # the read at line 4 reaches the copy at line 3 around the loop
    assert [(b[0], b[1]) for b in pending_uses(_BACKEDGE)] == [(4, 3)]
    assert pending_uses(_WAW_LDS) == []


# --- the kernels ------------------------------------------------------------------------------

def _sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


@pytest.fixture(scope="module")
def listings():
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    tmp = tempfile.mkdtemp(prefix="isa_")

    def build(src):
        out = os.path.join(tmp, src + ".s")
        r = subprocess.run([HIPCC, *FLAGS, os.path.join(CSRC, src), "-o", out], capture_output=True, text=True,
                           timeout=600)
        assert r.returncode == 0, "hipcc failed for %s:\n%s" % (src, r.stderr[-2000:])
        with open(out) as f:
            return src, f.read()

    with ThreadPoolExecutor(max_workers=4) as ex:
        res = dict(ex.map(build, _sources()))
    shutil.rmtree(tmp, ignore_errors=True)
    return res


@pytest.mark.parametrize("src", _sources())
def test_lds_reads_complete_before_use(listings, src):
    asm = listings[src]
    assert _kernels(asm), "no kernels found in %s" % src
    bad = pending_uses(asm)
    assert not bad, "%s: registers of pending LDS reads used (read line, use line, use): %s" % (src, bad[:10])

"""The oracle's own tests, run once more against a build of moe_ref.c with
AddressSanitizer and UndefinedBehaviorSanitizer (host code only: gcc, no GPU).

A read or write past a buffer, a use after free or an undefined integer
operation anywhere in the oracle ends that run with a sanitizer report, so a
pin that passes on the plain build cannot pass on memory it does not own."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = ["test_oracle_routing.py", "test_oracle_experts.py", "test_oracle_mxfp4.py", "test_oracle_mxfp8.py",
         "test_oracle_permute.py", "test_oracle_block.py"]


def _runtime(name):
    try:
        p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    except OSError:
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_tests_pass_under_asan_and_ubsan(tmp_path):
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("a preload is already set for this process; the sanitizer runtimes must load first")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not found")
    lib = str(tmp_path / "libmoe_ref_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                           "-fno-omit-frame-pointer", "-fopenmp", "-fPIC", "-shared", "-o", lib,
                           os.path.join(ROOT, "oracle", "moe_ref.c"), "-lm"])
    rep = str(tmp_path / "report")
    env = dict(os.environ, MOE_REF_LIB=lib, LD_PRELOAD=asan + ":" + ubsan,
               ASAN_OPTIONS="detect_leaks=0:log_path=" + rep, UBSAN_OPTIONS="log_path=" + rep,
               OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        *[os.path.join(ROOT, "tests", t) for t in TESTS]],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = sorted(p for p in os.listdir(tmp_path) if p.startswith("report"))
    text = "".join(open(os.path.join(tmp_path, p)).read()[:4000] for p in reports)
    assert not reports, "sanitizer report:\n" + text
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout

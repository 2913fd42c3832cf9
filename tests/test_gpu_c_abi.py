"""The layer driven from plain C (tests/c/moe_abi_check.c): HIP runtime
buffers, inputs from the seeded generator's C library, moe_forward through
include/moe.h with no Python in between, every output checked against the
C oracle on the GPU's picks, and the argument checks that precede any
launch.  The program is built by __graft_entry__.build()."""
import os
import subprocess

import pytest

from tests._parity import log

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c", "moe_abi_check")


@pytest.mark.parametrize("t_bf16,t_mxfp4", [(37, 16), (200, 150)], ids=["few-token", "mfma"])
def test_c_program_matches_the_oracle(t_bf16, t_mxfp4):
    assert os.path.exists(EXE), "tests/c/moe_abi_check is not built: run __graft_entry__.build()"
    log("C ABI program: bf16 T=%d, MXFP4 T=%d" % (t_bf16, t_mxfp4))
    r = subprocess.run([EXE, str(t_bf16), str(t_mxfp4)], capture_output=True, text=True, timeout=120)
    log(r.stdout.strip())
    assert r.returncode == 0, "exit %d\n%s\n%s" % (r.returncode, r.stdout, r.stderr)
    assert "all checks passed" in r.stdout

"""The C-ABI from a plain C program (tests/c_client/gemm_client.c, built by
the package's build step): HIP runtime memory and a stream, gemm_f16_nt and
gemm_f16_nt_rung through include/gemm_f16_nt.h, outputs checked bitwise on
the host against integer sums, an invalid call's status and untouched D."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c_client", "gemm_client")


def test_plain_c_client():
    assert os.path.exists(CLIENT), "not built: python -c 'import __graft_entry__ as g; g.build()'"
    print("[gpu] plain C client of the C-ABI", file=sys.stderr, flush=True)
    r = subprocess.run([CLIENT], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().splitlines()[-1] == "ok", r.stdout + r.stderr
    assert r.stdout.count("every output exact") == 4

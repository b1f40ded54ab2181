"""The plain C client of the boundary (tests/c_client/sv_client.c) on the GPU:
device memory from the HIP runtime, calls through include/spec_verify.h, no
Python or torch in the process.  It runs a greedy and a sampling call whose
results it works out itself (see the source)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c_client", "sv_client")


def test_c_client_on_the_gpu():
    if not os.path.exists(CLIENT):
        pytest.skip("tests/c_client/sv_client is built by __graft_entry__.build()")
    r = subprocess.run([CLIENT, "gpu"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed (gpu)" in r.stdout

"""The path driven from C alone: tests/c_client/qar_client.c (built by
__graft_entry__.build()) allocates with hipMalloc, calls libqar's C entry
points on its own stream and compares every result with the oracle's C
functions bit for bit."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_client", "qar_client")


def test_c_client_on_gpu():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is not built: run __graft_entry__.build()")
    print("running", EXE, flush=True)
    out = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, (out.returncode, out.stdout, out.stderr)
    assert out.stdout.strip() == "ok"

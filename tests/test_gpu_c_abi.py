"""The C ABI from plain C: tests/c_abi/decode_step.c (built by
__graft_entry__.build() with the host C compiler) allocates device buffers
with hipMalloc, runs a decode step through include/ksa.h and checks it by
properties that hold for any input (see the program's header)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "decode_step")


def test_decode_step_from_plain_c():
    assert os.path.exists(BIN), "tests/c_abi/decode_step is not built: run __graft_entry__.build()"
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("OK"), (r.returncode, r.stdout, r.stderr)

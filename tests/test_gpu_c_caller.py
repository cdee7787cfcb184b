"""The C ABI from a plain C program: tests/c/decode_step_caller.c (built by
the package build) fills qsa_tensor descriptors by hand over hipMalloc'd
buffers, calls qsa_decode_step on the null stream, checks a fail-closed
call, and compares the result with the oracle's C entry points.  No Python
or torch on the calling side; it runs as a child process."""

import os
import subprocess

import pytest

from gpu_util import banner

pytestmark = pytest.mark.gpu
EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "decode_step_caller")


def test_plain_c_caller():
    assert os.path.exists(EXE), "the C caller is built by __graft_entry__.build()"
    banner("plain C caller: qsa_decode_step through include/qsa.h")
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, res.stderr
    assert "c caller ok" in res.stdout

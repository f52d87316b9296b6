"""The C ABI from a plain C program (tests/abi_caller.c, built by
__graft_entry__.build()): device memory from hipMalloc, libfa2.so called
through include/fa2.h alone, results checked against closed forms inside the
program (K = 0: O is the mean of the live rows of V, LSE = ln of their
number), plus the error paths.  Runs as a child process of the test."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_bin", "abi_caller")


def test_c_caller():
    assert os.path.exists(BIN), "the C caller is not built: run __graft_entry__.build()"
    print("running", BIN, flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0 and "abi_caller: ok" in r.stdout, r.stdout + r.stderr

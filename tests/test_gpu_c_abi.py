"""The library called from C++ through include/bsa.h alone (tests/c/abi_check.cpp,
built next to libbsa.so by the package build): no Python binding, no torch
between the caller and the kernels.  Closed forms only -- V = 1 gives O = 1,
dO = 0 gives zero gradients -- plus the descriptor checks' error codes."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "block_sparse_varlen_amd", "abi_check")


def test_cpp_caller_through_the_c_abi():
    assert os.path.exists(EXE), "abi_check is built by the package build (block_sparse_varlen_amd/build.py)"
    print("c abi: running abi_check", flush=True)
    sys.stdout.flush()
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0 and "abi_check: ok" in r.stdout

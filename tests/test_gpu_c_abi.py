"""The C ABI used from C++ with no Python and no torch (tests/c_api/
c_abi_check.cpp, built by __graft_entry__.build()): hipMalloc'd buffers, a
HIP stream, AdamW (whole list, gradient release per tensor and in buckets),
Lion and SGD steps over a ragged list, every code and scale compared with the
oracle."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_api", "c_abi_check")


def test_c_consumer_matches_oracle():
    assert os.path.exists(BIN), "tests/c_api/c_abi_check is not built (run build())"
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    assert r.stdout.count("match the oracle") == 5

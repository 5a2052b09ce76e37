"""Build the HIP library libflashopt.so for gfx950 (in-tree, with hipcc).

Flags that the bit-exact arithmetic relies on:
  -ffp-contract=off                          no fused multiply-add contraction
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE binary32 division and sqrt
  -fno-gpu-flush-denormals-to-zero           binary32 subnormals kept
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed FP32 instructions
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "flashopt.hip")
LIB = os.path.join(PKG, "libflashopt.so")
ARCH = os.environ.get("FLASHOPT_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
]


TEST_SRC = os.path.join(ROOT, "tests", "hip", "codec_exhaustive.hip")
TEST_LIB = os.path.join(ROOT, "tests", "hip", "libcodec_exhaustive.so")


def build_test_lib(verbose: bool = False) -> str:
    """The exhaustive device check of the codec's short sequences (tests only)."""
    tmp = TEST_LIB + ".tmp"
    cmd = ["hipcc", *FLAGS, "-o", tmp, TEST_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, TEST_LIB)
    return TEST_LIB


C_CHECK_SRC = os.path.join(ROOT, "tests", "c_api", "c_abi_check.cpp")
C_CHECK_BIN = os.path.join(ROOT, "tests", "c_api", "c_abi_check")


def build_c_check(verbose: bool = False) -> str:
    """The C++ consumer of the C ABI the GPU tests run (tests only): host code
    linked against libflashopt.so and the oracle's liboracle.so."""
    tmp = C_CHECK_BIN + ".tmp"
    oracle_dir = os.path.join(ROOT, "oracle")
    cmd = ["hipcc", "-O2", "-std=c++17", "-Wall", "-I", os.path.join(ROOT, "include"),
           "-I", oracle_dir, "-o", tmp, C_CHECK_SRC, "-L", PKG, "-lflashopt", "-L", oracle_dir,
           "-loracle", "-Wl,-rpath,$ORIGIN/../../compressed_adamw_state_amd",
           "-Wl,-rpath,$ORIGIN/../../oracle"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, C_CHECK_BIN)
    return C_CHECK_BIN


def build(verbose: bool = False, extra=()) -> str:
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *FLAGS, *extra, "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])

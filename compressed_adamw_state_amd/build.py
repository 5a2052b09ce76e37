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
CSRC = os.path.join(PKG, "csrc")
# translation units of libflashopt.so: the fused step (hot path), the
# uncompressed kinds, one tensor's codec and state, the codec ablations, the
# measurement probes, the device schedules, the C ABI of tensor lists, and the
# step that allocates nothing
UNITS = ["step.hip", "step_fp32.hip", "tensor.hip", "ablation.hip", "probe.hip", "schedule.hip",
         "list.hip", "noalloc.hip"]
SOURCES = [os.path.join(CSRC, u) for u in UNITS] + [
    os.path.join(CSRC, h) for h in ("codec.hpp", "device.hpp", "host.hpp", "quant.hpp")]
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libflashopt.so")
ARCH = os.environ.get("FLASHOPT_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
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
    cmd = ["hipcc", *FLAGS, "-shared", "-o", tmp, TEST_SRC]
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
    """Compile every translation unit (in parallel) and link libflashopt.so."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, os.path.splitext(u)[0] + ".o") for u in UNITS]

    def compile_one(k):
        cmd = ["hipcc", *FLAGS, *extra, "-c", "-o", objs[k], os.path.join(CSRC, UNITS[k])]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)

    with ThreadPoolExecutor(min(len(UNITS), os.cpu_count() or 1)) as ex:
        list(ex.map(compile_one, range(len(UNITS))))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])

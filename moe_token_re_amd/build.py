"""Builds the HIP library libmoe_rerouting_v2.so in-tree, for gfx950.

The host checks (mrr_validate.cpp) are compiled by g++ with no HIP header; the
kernels and launchers (mrr_kernels.hip) by hipcc. Packed-fp32 instructions are
disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libmoe_rerouting_v2.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
BENCH_LIB_PATH = os.path.join(PKG, "libmrr_bench_copy.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-command-line-argument"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build_library(verbose: bool = False) -> str:
    """Compile and link the library; returns its path. Always recompiles."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    v_obj = os.path.join(BUILD_DIR, "mrr_validate.o")
    k_obj = os.path.join(BUILD_DIR, "mrr_kernels.o")
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Werror", "-I", INCLUDE,
          "-c", os.path.join(CSRC, "mrr_validate.cpp"), "-o", v_obj], verbose)
    _run([HIPCC, *HIP_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, "mrr_kernels.hip"),
          "-o", k_obj], verbose)
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, v_obj, k_obj], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def build_bench_copy(verbose: bool = False) -> str:
    """The benchmark's copy-ceiling kernel, in a library of its own."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = os.path.join(BUILD_DIR, "mrr_bench_copy.o")
    _run([HIPCC, *HIP_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, "mrr_bench_copy.hip"), "-o", obj],
         verbose)
    tmp = BENCH_LIB_PATH + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, obj], verbose)
    os.replace(tmp, BENCH_LIB_PATH)
    return BENCH_LIB_PATH


def build_all(verbose: bool = False):
    return build_library(verbose), build_bench_copy(verbose)


if __name__ == "__main__":
    print(build_all(verbose="-v" in sys.argv))

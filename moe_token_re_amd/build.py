"""Builds the HIP library libmoe_rerouting_v2.so in-tree, for gfx950.

The host checks (mrr_validate.cpp) are compiled by g++ with no HIP header; the
kernel files (mrr_offsets.hip, mrr_gather.hip, mrr_fused.hip,
mrr_one_launch.hip) and the entry points (mrr_entry.hip) by hipcc, in
parallel. Packed-fp32 instructions are
disabled for all device code.
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

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


def source_files():
    """Every source the library is built from: the kernels, launchers and host
    checks under csrc/ and the public header."""
    names = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h", ".cpp")) and not f.startswith("mrr_bench"))
    return [os.path.join(CSRC, f) for f in names] + [os.path.join(INCLUDE, "moe_rerouting_v2.h")]


def source_hash() -> str:
    """16 hex digits of SHA-256 over the sources' names and bytes. The build
    compiles it into the library (mrr_source_hash()), and the loader compares
    the two, so a library built from other sources is never run as this one."""
    h = hashlib.sha256()
    for p in source_files():
        h.update(os.path.basename(p).encode() + b"\0")
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


HIP_SOURCES = ("mrr_offsets.hip", "mrr_gather.hip", "mrr_fused.hip", "mrr_one_launch.hip", "mrr_entry.hip")


def build_library(verbose: bool = False) -> str:
    """Compile and link the library; returns its path. Always recompiles."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    v_obj = os.path.join(BUILD_DIR, "mrr_validate.o")
    cmds = [["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Werror", "-I", INCLUDE,
             f'-DMRR_SOURCE_HASH="{source_hash()}"',
             "-c", os.path.join(CSRC, "mrr_validate.cpp"), "-o", v_obj]]
    objs = [v_obj]
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmds.append([HIPCC, *HIP_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as pool:
        for f in [pool.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
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

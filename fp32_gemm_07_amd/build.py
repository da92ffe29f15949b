"""Compile libgemm.so (HIP, gfx950 only) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libgemm.so")
SOURCES = [os.path.join(CSRC, "gemm_api.hip")]
DEPENDS = SOURCES + [os.path.join(CSRC, "gemm_kernels.hpp"), os.path.join(CSRC, "ladder_kernels.hpp"),
                     os.path.join(INCLUDE, "gemm.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from forming packed FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False, extra_flags=None) -> str:
    """Always recompile; returns the path of the built library."""
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, *HIPCC_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)

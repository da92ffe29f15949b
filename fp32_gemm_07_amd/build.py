"""Compile libgemm.so (HIP, gfx950 only) in-tree with hipcc."""
from __future__ import annotations

import os
import re
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


# The compiler's per-kernel resource report (one remark per line, after a
# "Function Name" line) is read to refuse kernels that spill to scratch memory.
RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"
_FUNC = re.compile(r"remark: Function Name: (\S+)")
_FIELD = re.compile(r"remark:\s+(ScratchSize \[bytes/lane\]|VGPRs Spill|SGPRs Spill|VGPRs|AGPRs): (\d+)")


class ScratchError(RuntimeError):
    """A kernel of the library uses scratch memory (registers spilled to memory)."""


def kernel_resources(remarks: str) -> dict:
    """Kernel symbol -> {field: value} from the resource-usage remarks."""
    out, cur = {}, None
    for line in remarks.splitlines():
        m = _FUNC.search(line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = _FIELD.search(line)
        if m and cur is not None:
            cur[m.group(1)] = int(m.group(2))
    return out


def spilling_kernels(resources: dict) -> dict:
    """Kernels with scratch memory per lane or VGPRs spilled (SGPRs spilled into
    VGPR lanes cost no memory and are allowed)."""
    return {k: v for k, v in resources.items()
            if v.get("ScratchSize [bytes/lane]", 0) > 0 or v.get("VGPRs Spill", 0) > 0}


def build(verbose: bool = False, extra_flags=None) -> str:
    """Always recompile; returns the path of the built library. Raises
    ScratchError (and keeps the previous library) if any kernel spills."""
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, *HIPCC_FLAGS, RESOURCE_REMARKS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC,
           *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    diagnostics = "\n".join(l for l in res.stderr.splitlines()
                            if "remark" not in l and "packed-fp32-ops" not in l
                            and not l.strip().startswith("|") and not re.match(r"^\s*\d+ \|", l))
    if res.returncode != 0:
        sys.stderr.write(res.stderr)
        raise subprocess.CalledProcessError(res.returncode, cmd)
    if verbose and diagnostics.strip():
        print(diagnostics, flush=True)
    resources = kernel_resources(res.stderr)
    if not resources:
        raise RuntimeError("no kernel resource report in the compiler output")
    bad = spilling_kernels(resources)
    if bad:
        os.remove(tmp)
        raise ScratchError("kernels using scratch memory: " +
                           "; ".join(f"{k}: {v}" for k, v in sorted(bad.items())))
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"{len(resources)} kernels, none using scratch memory", flush=True)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)

"""Compile libgemm.so (HIP, gfx950 only) in-tree with hipcc."""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libgemm.so")
SOURCES = [os.path.join(CSRC, "gemm_api.hip"), os.path.join(CSRC, "gemm_dma.hip")]
DEPENDS = SOURCES + [os.path.join(CSRC, "gemm_kernels.hpp"), os.path.join(CSRC, "ladder_kernels.hpp"),
                     os.path.join(CSRC, "dma_launch.hpp"), os.path.join(INCLUDE, "gemm.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep the compiler from forming packed FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]
# Per source: the copy-fed kernels' launches get their first 12 kernel
# arguments in scalar registers at wave launch (their tile order and first
# copies need nothing else; a 256-byte entry block loads them the ordinary way
# where the firmware does not preload). The register-staged kernels of
# gemm_api.hip, at the edge of their register budget, would spill with it.
SOURCE_FLAGS = {
    "gemm_dma.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=12"],
}


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
    objdir = tempfile.mkdtemp(prefix="libgemm_objs_")
    try:
        jobs = []
        for src in SOURCES:   # each source its own object, compiled side by side
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            cmd = [HIPCC, *HIPCC_FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []), RESOURCE_REMARKS,
                   *(extra_flags or []), "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            jobs.append((cmd, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                    stderr=subprocess.PIPE, text=True)))
        remarks = []
        for cmd, _, proc in jobs:
            _, err = proc.communicate()
            if proc.returncode != 0:
                sys.stderr.write(err)
                raise subprocess.CalledProcessError(proc.returncode, cmd)
            remarks.append(err)
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for _, o, _ in jobs], "-o", tmp]
        res = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stderr)
            raise subprocess.CalledProcessError(res.returncode, link)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    stderr = "\n".join(remarks)
    diagnostics = "\n".join(l for l in stderr.splitlines()
                            if "remark" not in l and "packed-fp32-ops" not in l
                            and not l.strip().startswith("|") and not re.match(r"^\s*\d+ \|", l))
    if verbose and diagnostics.strip():
        print(diagnostics, flush=True)
    resources = kernel_resources(stderr)
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

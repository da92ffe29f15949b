"""ctypes binding of libgemm (the C ABI in include/gemm.h), same names, marshalling only.

Every entry takes device pointers as Python ints (or anything with a
``data_ptr()`` method, such as a torch tensor on the GPU) and a HIP stream
handle as an int (``torch.cuda.current_stream().cuda_stream``; 0 = null
stream). Nonzero statuses raise ``GemmError``; nothing here computes.

The library must have been built (``fp32_gemm_07_amd.build.build()``): a
missing library raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

GEMM_OK = 0
GEMM_ERR_INVALID_DIM = 1
GEMM_ERR_NULL_PTR = 2
GEMM_ERR_ALIAS = 3
GEMM_ERR_WORKSPACE = 4
GEMM_ERR_INVALID_PLAN = 5
GEMM_ERR_HIP = 6
GEMM_ERR_UNSUPPORTED_DEVICE = 7
GEMM_ERR_CAPTURING = 8
GEMM_ERR_SCRATCH_LIMIT = 9

GEMM_KERNEL_AUTO = 0
GEMM_KERNEL_MFMA_256x256 = 1
GEMM_KERNEL_MFMA_256x128 = 2
GEMM_KERNEL_MFMA_128x128 = 3
GEMM_KERNEL_MFMA_64x64 = 4
GEMM_KERNEL_MFMA_256x256_W8 = 5
GEMM_KERNEL_VALU_64x64 = 10
GEMM_KERNEL_MFMA16_256x128 = 13
GEMM_KERNEL_MFMA16_128x128 = 14
GEMM_KERNEL_MFMA16_64x64 = 15
GEMM_KERNEL_MFMA16_128x128_K16 = 17
GEMM_KERNEL_MFMA16_256x128_K16 = 18
GEMM_KERNEL_MFMA_128x128_W1 = 19
GEMM_KERNEL_MFMA_64x64_W1 = 21
GEMM_KERNEL_DMA32_256x256_W8 = 30
GEMM_KERNEL_DMA32_128x128_W4 = 33
GEMM_KERNEL_DMA16_128x128_W4 = 34
GEMM_KERNEL_DMA32_256x256_W8_S3 = 35
GEMM_KERNEL_DMA16_64x64 = 36
GEMM_KERNEL_DMA32_64x64 = 37
GEMM_KERNEL_DMA16_128x64 = 38
GEMM_KERNEL_DMA32_128x128_W8 = 39
GEMM_KERNEL_DMA32_64x64_S3 = 45
GEMM_KERNEL_DMA32_128x128_W8_S3 = 46
GEMM_KERNEL_DMA16_96x96_S3 = 47
GEMM_KERNEL_LADDER_V0 = 40
GEMM_KERNEL_LADDER_V1 = 41
GEMM_KERNEL_LADDER_V2 = 42
GEMM_KERNEL_LADDER_V3 = 43

KERNELS = {
    "mfma32_256x256": GEMM_KERNEL_MFMA_256x256,
    "mfma32_256x256_w8": GEMM_KERNEL_MFMA_256x256_W8,
    "mfma32_256x128": GEMM_KERNEL_MFMA_256x128,
    "mfma32_128x128": GEMM_KERNEL_MFMA_128x128,
    "mfma32_64x64": GEMM_KERNEL_MFMA_64x64,
    "mfma16_256x128": GEMM_KERNEL_MFMA16_256x128,
    "mfma16_128x128": GEMM_KERNEL_MFMA16_128x128,
    "mfma16_64x64": GEMM_KERNEL_MFMA16_64x64,
    "mfma16_128x128_k16": GEMM_KERNEL_MFMA16_128x128_K16,
    "mfma16_256x128_k16": GEMM_KERNEL_MFMA16_256x128_K16,
    "mfma32_128x128_w1": GEMM_KERNEL_MFMA_128x128_W1,
    "mfma32_64x64_w1": GEMM_KERNEL_MFMA_64x64_W1,
    "dma32_256x256_w8": GEMM_KERNEL_DMA32_256x256_W8,
    "dma32_128x128_w4": GEMM_KERNEL_DMA32_128x128_W4,
    "dma16_128x128_w4": GEMM_KERNEL_DMA16_128x128_W4,
    "dma32_256x256_w8_s3": GEMM_KERNEL_DMA32_256x256_W8_S3,
    "dma16_64x64": GEMM_KERNEL_DMA16_64x64,
    "dma32_64x64": GEMM_KERNEL_DMA32_64x64,
    "dma16_128x64": GEMM_KERNEL_DMA16_128x64,
    "dma32_128x128_w8": GEMM_KERNEL_DMA32_128x128_W8,
    "dma32_64x64_s3": GEMM_KERNEL_DMA32_64x64_S3,
    "dma32_128x128_w8_s3": GEMM_KERNEL_DMA32_128x128_W8_S3,
    "dma16_96x96_s3": GEMM_KERNEL_DMA16_96x96_S3,
    "valu_64x64": GEMM_KERNEL_VALU_64x64,
    "ladder_v0": GEMM_KERNEL_LADDER_V0,
    "ladder_v1": GEMM_KERNEL_LADDER_V1,
    "ladder_v2": GEMM_KERNEL_LADDER_V2,
    "ladder_v3": GEMM_KERNEL_LADDER_V3,
}

# Every symbol include/gemm.h declares.
EXPORTS = (
    "gemm_f32", "gemm_f32_noalloc", "gemm_f32_noalloc_scratch_bytes", "gemm_f32_workspace_bytes",
    "gemm_f32_ex", "gemm_f32_plan", "gemm_f32_plan_cus",
    "gemm_f32_plan_workspace_bytes", "gemm_f32_with_plan", "gemm_f32_general",
    "gemm_f32_general_workspace_bytes", "gemm_kernel_name", "gemm_status_string",
    "gemm_last_hip_error",
)


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        text = gemm_status_string(status)
        if status == GEMM_ERR_HIP:
            text += f" (hipError_t {gemm_last_hip_error()})"
        super().__init__(f"{where}: {text} [status {status}]")


class gemm_plan_t(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("split_k", ctypes.c_int),
                ("k_chunk", ctypes.c_int), ("split_tail", ctypes.c_int)]

    def __repr__(self):
        return (f"gemm_plan_t(kernel={gemm_kernel_name(self.kernel)}, split_k={self.split_k}, "
                f"k_chunk={self.k_chunk}, split_tail={self.split_tail})")


_lib = None


def _share_hip_runtime() -> None:
    """Make libgemm use the HIP runtime the caller's memory and streams come from.

    PyTorch-ROCm wheels bundle their own libamdhip64 (and HSA runtime) under
    the soname libamdhip64.so.7. A process that ends up with two HIP runtimes
    cannot use the GPU from the second one (device enumeration fails), and
    pointers and streams of one are meaningless to the other. libgemm names
    its runtime only by soname, and the dynamic linker resolves a soname to a
    library already loaded under it, so loading torch first makes libgemm
    bind to torch's runtime. Without torch installed, the system ROCm runtime
    is used.
    """
    try:
        import torch  # noqa: F401
    except ImportError:
        pass


def library_path() -> str:
    return LIB_PATH


def load():
    """Load libgemm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libgemm is not built ({LIB_PATH} missing); run "
                               "fp32_gemm_07_amd.build.build() first")
        _share_hip_runtime()
        lib = ctypes.CDLL(LIB_PATH)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        plan_p = ctypes.POINTER(gemm_plan_t)
        lib.gemm_f32.argtypes = [vp, vp, vp, i, i, i, vp]
        lib.gemm_f32.restype = i
        lib.gemm_f32_noalloc.argtypes = [vp, vp, vp, i, i, i, vp]
        lib.gemm_f32_noalloc.restype = i
        lib.gemm_f32_noalloc_scratch_bytes.argtypes = []
        lib.gemm_f32_noalloc_scratch_bytes.restype = sz
        lib.gemm_f32_workspace_bytes.argtypes = [i, i, i]
        lib.gemm_f32_workspace_bytes.restype = sz
        lib.gemm_f32_ex.argtypes = [vp, vp, vp, i, i, i, vp, sz, vp]
        lib.gemm_f32_ex.restype = i
        lib.gemm_f32_plan.argtypes = [i, i, i, plan_p]
        lib.gemm_f32_plan.restype = i
        lib.gemm_f32_plan_cus.argtypes = [i, i, i, i, plan_p]
        lib.gemm_f32_plan_cus.restype = i
        lib.gemm_f32_plan_workspace_bytes.argtypes = [i, i, i, plan_p]
        lib.gemm_f32_plan_workspace_bytes.restype = sz
        lib.gemm_f32_with_plan.argtypes = [vp, vp, vp, i, i, i, plan_p, vp, sz, vp]
        lib.gemm_f32_with_plan.restype = i
        f = ctypes.c_float
        lib.gemm_f32_general.argtypes = [i, i, i, i, i, f, vp, i, vp, i, f, vp, i, vp, sz, vp]
        lib.gemm_f32_general.restype = i
        lib.gemm_f32_general_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
        lib.gemm_f32_general_workspace_bytes.restype = sz
        lib.gemm_kernel_name.argtypes = [i]
        lib.gemm_kernel_name.restype = ctypes.c_char_p
        lib.gemm_status_string.argtypes = [i]
        lib.gemm_status_string.restype = ctypes.c_char_p
        lib.gemm_last_hip_error.argtypes = []
        lib.gemm_last_hip_error.restype = i
        _lib = lib
    return _lib


def _addr(p) -> int:
    if p is None:
        return 0
    if hasattr(p, "data_ptr"):
        return int(p.data_ptr())
    return int(p)


def _check(status: int, where: str) -> int:
    if status != GEMM_OK:
        raise GemmError(status, where)
    return status


def gemm_f32(A, B, C, M: int, N: int, K: int, stream: int = 0) -> None:
    _check(load().gemm_f32(_addr(A), _addr(B), _addr(C), M, N, K, stream or None), "gemm_f32")


def gemm_f32_noalloc(A, B, C, M: int, N: int, K: int, stream: int = 0) -> None:
    _check(load().gemm_f32_noalloc(_addr(A), _addr(B), _addr(C), M, N, K, stream or None),
           "gemm_f32_noalloc")


def gemm_f32_noalloc_scratch_bytes() -> int:
    return int(load().gemm_f32_noalloc_scratch_bytes())


def gemm_f32_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(load().gemm_f32_workspace_bytes(M, N, K))


def gemm_f32_ex(A, B, C, M: int, N: int, K: int, workspace, workspace_bytes: int,
                stream: int = 0) -> None:
    _check(load().gemm_f32_ex(_addr(A), _addr(B), _addr(C), M, N, K, _addr(workspace) or None,
                              workspace_bytes, stream or None), "gemm_f32_ex")


def gemm_f32_plan(M: int, N: int, K: int) -> gemm_plan_t:
    p = gemm_plan_t()
    _check(load().gemm_f32_plan(M, N, K, ctypes.byref(p)), "gemm_f32_plan")
    return p


def gemm_f32_plan_cus(M: int, N: int, K: int, num_cus: int) -> gemm_plan_t:
    p = gemm_plan_t()
    _check(load().gemm_f32_plan_cus(M, N, K, num_cus, ctypes.byref(p)), "gemm_f32_plan_cus")
    return p


def make_plan(kernel: int, split_k: int = 1, split_tail: bool = False) -> gemm_plan_t:
    """An explicit plan; split_tail splits only the tiles of the last, partial
    round of one tile per CU (copy-fed kernels only)."""
    return gemm_plan_t(kernel, split_k, 0, int(split_tail))


def gemm_f32_plan_workspace_bytes(M: int, N: int, K: int, plan: gemm_plan_t) -> int:
    return int(load().gemm_f32_plan_workspace_bytes(M, N, K, ctypes.byref(plan)))


def gemm_f32_with_plan(A, B, C, M: int, N: int, K: int, plan: gemm_plan_t, workspace=None,
                       workspace_bytes: int = 0, stream: int = 0) -> None:
    _check(load().gemm_f32_with_plan(_addr(A), _addr(B), _addr(C), M, N, K, ctypes.byref(plan),
                                     _addr(workspace) or None, workspace_bytes, stream or None),
           "gemm_f32_with_plan")


def gemm_f32_general(trans_a: bool, trans_b: bool, M: int, N: int, K: int, alpha: float, A,
                     lda: int, B, ldb: int, beta: float, C, ldc: int, workspace=None,
                     workspace_bytes: int = 0, stream: int = 0) -> None:
    _check(load().gemm_f32_general(int(bool(trans_a)), int(bool(trans_b)), M, N, K, alpha,
                                   _addr(A) or None, lda, _addr(B) or None, ldb, beta,
                                   _addr(C) or None, ldc, _addr(workspace) or None,
                                   workspace_bytes, stream or None), "gemm_f32_general")


def gemm_f32_general_workspace_bytes(trans_a: bool, trans_b: bool, M: int, N: int, K: int,
                                     lda: int, ldb: int) -> int:
    return int(load().gemm_f32_general_workspace_bytes(int(bool(trans_a)), int(bool(trans_b)),
                                                       M, N, K, lda, ldb))


def gemm_kernel_name(kernel: int) -> str:
    return load().gemm_kernel_name(kernel).decode()


def gemm_status_string(status: int) -> str:
    return load().gemm_status_string(status).decode()


def gemm_last_hip_error() -> int:
    return int(load().gemm_last_hip_error())


def raw_status(fn: str, *args) -> int:
    """Call an entry point and return its raw status (for tests of the error paths)."""
    return int(getattr(load(), fn)(*args))

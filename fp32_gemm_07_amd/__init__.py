"""MI355X-native row-major FP32 GEMM (C = A x B) behind a C ABI (include/gemm.h).

``fp32_gemm_07_amd.binding`` is the ctypes binding of libgemm.so;
``fp32_gemm_07_amd.build`` compiles it for gfx950; ``fp32_gemm_07_amd.roofline``
holds the work and peak figures the bench reports against.
"""
from . import binding  # noqa: F401  (loads lazily; raises on first use if unbuilt)

__all__ = ["binding"]

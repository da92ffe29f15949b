// Launch of the copy-fed kernels (mfma_dma_gemm_kernel), compiled in a
// translation unit of its own (gemm_dma.hip): that one is built with the
// kernel arguments preloaded into scalar registers, which the register-staged
// kernels of gemm_api.hip, at the edge of their register budget, cannot
// afford.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_kernels.hpp"

namespace gemm {

// One launch, as plain data: the product C <- alpha * op(A) op(B) + beta * C
// (op = transpose where ta / tb), or with a split the partial products into
// the workspace slabs ws + s * slab; the tile order in the kernel's scalar
// form; workgroups = whole tiles + split tiles x splits.
struct DmaLaunch {
  const float *A, *B;
  float *C, *ws;
  int M, N, K, lda, ldb, ldc;
  float alpha, beta;
  bool ta, tb;
  int k_chunk;
  long long slab;
  KernelOrder order;
  long long workgroups;
};

// Launches copy-fed kernel `kernel` (a GEMM_KERNEL_DMA* id). False, with
// nothing launched, for any other id and for transposed operands on a
// configuration built for op = identity only. The caller has checked that
// the operand offsets fit in 32 bits.
bool launch_dma_kernel(int kernel, const DmaLaunch &d, hipStream_t stream);

}  // namespace gemm

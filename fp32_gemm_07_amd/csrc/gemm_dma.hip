// The copy-fed kernels' launches (see dma_launch.hpp). Built with the first
// 12 kernel arguments preloaded into scalar registers.
#include "gemm.h"
#include "dma_launch.hpp"

namespace gemm {
namespace {

template <int MI, int BM, int BN, int BK, int WAVES_M, int WAVES_N, int NS, int WPE, bool A_KM,
          bool B_KM>
void launch_t(const DmaLaunch &d, hipStream_t stream) {
  const KernelOrder &o = d.order;
  hipLaunchKernelGGL(
      (mfma_dma_gemm_kernel<MI, BM, BN, BK, WAVES_M, WAVES_N, NS, 4, WPE, A_KM, B_KM>),
      dim3(static_cast<unsigned>(d.workgroups)), dim3(64 * WAVES_M * WAVES_N), 0, stream, d.A, d.B,
      d.M, d.N, d.K, d.lda, d.ldb, o.dp_tiles, o.group_mul, o.rows_mul, o.shifts, o.splits, d.C,
      d.ws, d.ldc, d.alpha, d.beta, d.k_chunk, d.slab);
}

// ALL_ORDERS: the configuration is built for transposed operands too (the
// planner's five kernels); the others take op(A) = A, op(B) = B only.
template <int MI, int BM, int BN, int BK, int WAVES_M, int WAVES_N, int NS, int WPE,
          bool ALL_ORDERS>
bool launch_orders(const DmaLaunch &d, hipStream_t stream) {
#define LGEMM_DMA(AK, BKM) launch_t<MI, BM, BN, BK, WAVES_M, WAVES_N, NS, WPE, AK, BKM>(d, stream)
  if (!d.ta && !d.tb) {
    LGEMM_DMA(true, false);
    return true;
  }
  if constexpr (ALL_ORDERS) {
    if (d.ta && !d.tb) LGEMM_DMA(false, false);
    else if (!d.ta && d.tb) LGEMM_DMA(true, true);
    else LGEMM_DMA(false, true);
    return true;
  }
#undef LGEMM_DMA
  return false;
}

}  // namespace

bool launch_dma_kernel(int kernel, const DmaLaunch &d, hipStream_t stream) {
  switch (kernel) {
    case GEMM_KERNEL_DMA32_256x256_W8:
      return launch_orders<32, 256, 256, 16, 2, 4, 4, 2, false>(d, stream);
    case GEMM_KERNEL_DMA32_256x256_W8_S3:
      return launch_orders<32, 256, 256, 16, 2, 4, 3, 2, true>(d, stream);
    case GEMM_KERNEL_DMA32_128x128_W4:
      return launch_orders<32, 128, 128, 16, 2, 2, 4, 2, true>(d, stream);
    case GEMM_KERNEL_DMA16_128x128_W4:
      return launch_orders<16, 128, 128, 16, 2, 2, 4, 2, false>(d, stream);
    case GEMM_KERNEL_DMA16_64x64:
      return launch_orders<16, 64, 64, 32, 2, 2, 4, 2, false>(d, stream);
    case GEMM_KERNEL_DMA32_64x64:
      return launch_orders<32, 64, 64, 16, 2, 2, 4, 2, false>(d, stream);
    case GEMM_KERNEL_DMA16_128x64:
      // 96 KiB of LDS: one workgroup, so one wave per SIMD, per CU; built for
      // that (asking for two would only constrain the register allocator)
      return launch_orders<16, 128, 64, 32, 2, 2, 4, 1, false>(d, stream);
    case GEMM_KERNEL_DMA32_128x128_W8:
      return launch_orders<32, 128, 128, 16, 2, 4, 4, 2, false>(d, stream);
    case GEMM_KERNEL_DMA32_128x128_W8_S3:
      return launch_orders<32, 128, 128, 16, 2, 4, 3, 2, true>(d, stream);
    case GEMM_KERNEL_DMA32_64x64_S3:
      return launch_orders<32, 64, 64, 16, 2, 2, 3, 2, true>(d, stream);
    case GEMM_KERNEL_DMA16_96x96_S3:
      return launch_orders<16, 96, 96, 32, 2, 2, 3, 2, true>(d, stream);
  }
  return false;
}

}  // namespace gemm

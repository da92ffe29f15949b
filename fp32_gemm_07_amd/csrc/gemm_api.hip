// Host side of libgemm: argument checks, planner, workspace, launches.
// The C ABI is declared (and documented) in include/gemm.h.
#include "gemm.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstring>
#include <cmath>
#include <mutex>

#include "gemm_kernels.hpp"
#include "ladder_kernels.hpp"

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return GEMM_ERR_HIP;
}

constexpr int kNumCus = 256;

// ---------------------------------------------------------------------------
// Kernel configurations.
struct KernelInfo {
  int id;
  int bm, bn, bk;
  const char *name;
};

constexpr KernelInfo kKernels[] = {
    {GEMM_KERNEL_MFMA_256x256, 256, 256, 16, "mfma32_f32_256x256x16"},
    {GEMM_KERNEL_MFMA_256x256_W8, 256, 256, 16, "mfma32_f32_256x256x16_w8"},
    {GEMM_KERNEL_MFMA_256x128, 256, 128, 16, "mfma32_f32_256x128x16"},
    {GEMM_KERNEL_MFMA_128x128, 128, 128, 16, "mfma32_f32_128x128x16"},
    {GEMM_KERNEL_MFMA_64x64, 64, 64, 16, "mfma32_f32_64x64x16"},
    {GEMM_KERNEL_MFMA16_256x256, 256, 256, 32, "mfma16_f32_256x256x32"},
    {GEMM_KERNEL_MFMA16_256x256_W8, 256, 256, 32, "mfma16_f32_256x256x32_w8"},
    {GEMM_KERNEL_MFMA16_256x128, 256, 128, 32, "mfma16_f32_256x128x32"},
    {GEMM_KERNEL_MFMA16_128x128, 128, 128, 32, "mfma16_f32_128x128x32"},
    {GEMM_KERNEL_MFMA16_64x64, 64, 64, 32, "mfma16_f32_64x64x32"},
    {GEMM_KERNEL_MFMA16_256x256_K16, 256, 256, 16, "mfma16_f32_256x256x16"},
    {GEMM_KERNEL_MFMA16_128x128_K16, 128, 128, 16, "mfma16_f32_128x128x16"},
    {GEMM_KERNEL_MFMA16_256x128_K16, 256, 128, 16, "mfma16_f32_256x128x16"},
    {GEMM_KERNEL_MFMA_128x128_W1, 128, 128, 16, "mfma32_f32_128x128x16_w1"},
    {GEMM_KERNEL_MFMA16_128x128_W1, 128, 128, 16, "mfma16_f32_128x128x16_w1"},
    {GEMM_KERNEL_MFMA_64x64_W1, 64, 64, 16, "mfma32_f32_64x64x16_w1"},
    {GEMM_KERNEL_VALU_64x64, 64, 64, 16, "valu_f32_64x64x16"},
    {GEMM_KERNEL_DMA32_256x256_W8, 256, 256, 16, "dma_mfma32_f32_256x256x16_w8_s4"},
    {GEMM_KERNEL_DMA16_256x256_W8, 256, 256, 16, "dma_mfma16_f32_256x256x16_w8_s4"},
    {GEMM_KERNEL_DMA32_128x128_W4, 128, 128, 16, "dma_mfma32_f32_128x128x16_w4_s4"},
    {GEMM_KERNEL_DMA16_128x128_W4, 128, 128, 16, "dma_mfma16_f32_128x128x16_w4_s4"},
    {GEMM_KERNEL_DMA32_256x256_W8_S3, 256, 256, 16, "dma_mfma32_f32_256x256x16_w8_s3"},
    {GEMM_KERNEL_DMA16_64x64, 64, 64, 32, "dma_mfma16_f32_64x64x32_w4_s4"},
    {GEMM_KERNEL_DMA32_64x64, 64, 64, 16, "dma_mfma32_f32_64x64x16_w4_s4"},
    {GEMM_KERNEL_DMA16_128x64, 128, 64, 32, "dma_mfma16_f32_128x64x32_w4_s4"},
    {GEMM_KERNEL_LADDER_V0, 16, 16, 16, "ladder_v0_naive_rows_along_lanes"},
    {GEMM_KERNEL_LADDER_V1, 16, 16, 16, "ladder_v1_naive_cols_along_lanes"},
    {GEMM_KERNEL_LADDER_V2, 16, 16, 16, "ladder_v2_lds_16x16x16"},
    {GEMM_KERNEL_LADDER_V3, 16, 64, 16, "ladder_v3_lds_16x64x16_tn4"},
};

const KernelInfo *find_kernel(int id) {
  for (const auto &k : kKernels)
    if (k.id == id) return &k;
  return nullptr;
}

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

struct Resolved {
  const KernelInfo *k;
  int splits;     // number of K ranges actually launched (>= 1)
  int k_chunk;    // length of each K range
  long long tiles_m, tiles_n;
};

// Turn (kernel, requested split) into launch geometry. The split is clamped
// to the number of K steps; every range then holds at least one element.
bool resolve(int M, int N, int K, int kernel, int split_req, Resolved *out) {
  const KernelInfo *k = find_kernel(kernel);
  if (!k || split_req < 1) return false;
  out->k = k;
  out->tiles_m = ceil_div(M, k->bm);
  out->tiles_n = ceil_div(N, k->bn);
  const long long ksteps = std::max<long long>(1, ceil_div(K, k->bk));
  const long long s = std::min<long long>(split_req, ksteps);
  const long long chunk = ceil_div(ceil_div(std::max(K, 1), s), k->bk) * k->bk;
  out->k_chunk = static_cast<int>(std::min<long long>(chunk, INT_MAX));
  out->splits = static_cast<int>(K > 0 ? ceil_div(K, out->k_chunk) : 1);
  return true;
}

size_t workspace_for(int M, int N, const Resolved &r) {
  return r.splits > 1 ? sizeof(float) * (size_t)r.splits * (size_t)M * (size_t)N : 0;
}

// The planner: a cost model over three copy-fed kernels and power-of-two
// K splits, fitted to timings of those kernels over square, wide, long-K and
// ragged shapes on one MI355X. A CU works through its share of a launch's
// workgroups (at most n = ceil(workgroups / CUs) of them), so a launch costs
//   n * (2 * BM * BN * k_chunk / (rate_cu * eff) + per_wg) + fixed
// with rate_cu = 256 FLOP/clk at 2.38 GHz and eff, per_wg (prologue and
// epilogue of one workgroup) and fixed (launch, clock skew between XCDs)
// per kernel below. Splitting K adds the partial sums (S slabs written and
// read, C written), which stay in the last-level cache at these sizes,
// at about 8 TB/s plus a fixed cost for the extra launch; and no launch is
// cheaper than moving A, B and C once at about 5 TB/s. Workspace is capped
// at 1 GiB.
struct PlanCandidate {
  int kernel;
  double eff;
  double per_wg_us;
  double fixed_us;
};
constexpr PlanCandidate kPlanCandidates[] = {
    {GEMM_KERNEL_DMA32_256x256_W8_S3, 0.966, 11.9, 5.6},
    {GEMM_KERNEL_DMA32_128x128_W4, 0.955, 4.8, 5.1},
    {GEMM_KERNEL_DMA32_64x64, 0.91, 1.2, 6.5},
};
constexpr double kRateCuFlopPerUs = 256.0 * 2.38e3;   // FLOP per microsecond per CU
constexpr double kReduceBytesPerUs = 8.0e6;           // split-K partial sums
constexpr double kReduceFixedUs = 6.0;
constexpr double kMaxWorkspaceBytes = 1024.0 * 1024.0 * 1024.0;
constexpr double kHbmBytesPerUs = 5.0e6;

double plan_cost_us(int M, int N, int K, const PlanCandidate &c, int split, int *splits_out) {
  Resolved r;
  if (!resolve(M, N, K, c.kernel, split, &r)) return 1e30;
  const double wg = static_cast<double>(r.tiles_m * r.tiles_n * r.splits);
  const double per_cu = std::ceil(wg / kNumCus);
  const double flop = 2.0 * r.k->bm * r.k->bn * static_cast<double>(r.k_chunk);
  double us = per_cu * (flop / (kRateCuFlopPerUs * c.eff) + c.per_wg_us) + c.fixed_us;
  if (r.splits > 1) {
    const double slab = 4.0 * M * static_cast<double>(N);
    if (slab * r.splits > kMaxWorkspaceBytes) return 1e30;
    us += (2.0 * r.splits + 1.0) * slab / kReduceBytesPerUs + kReduceFixedUs;
  }
  // No launch beats reading A and B and writing C once (about 5 TB/s).
  const double bytes = 4.0 * (static_cast<double>(M) * K + static_cast<double>(K) * N +
                              static_cast<double>(M) * N);
  *splits_out = r.splits;
  return std::max(us, bytes / kHbmBytesPerUs + c.fixed_us);
}

void plan(int M, int N, int K, int *kernel, int *split) {
  *kernel = kPlanCandidates[0].kernel;
  *split = 1;
  double best = 1e30;
  for (const PlanCandidate &c : kPlanCandidates) {
    for (int s = 1; s <= 64; s *= 2) {
      if (s > 1 && K / s < 256) break;   // each K range keeps >= 256 elements
      int launched = 1;
      const double us = plan_cost_us(M, N, K, c, s, &launched);
      if (launched < s) break;           // fewer K steps than ranges asked for
      // Ties (within 1%) go to the candidate seen first: bigger tiles, fewer splits.
      if (us < best * 0.99) {
        best = us;
        *kernel = c.kernel;
        *split = s;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Device check (once per device): the code objects are built for gfx950 only.
std::mutex g_mu;
constexpr int kMaxDevices = 64;
int g_dev_ok[kMaxDevices];            // 0 unknown, 1 gfx950, -1 other
void *g_ws[kMaxDevices];
size_t g_ws_bytes[kMaxDevices];

int check_device(int *dev_out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return GEMM_ERR_UNSUPPORTED_DEVICE;
  *dev_out = dev;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_dev_ok[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e);
    g_dev_ok[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
  }
  return g_dev_ok[dev] == 1 ? GEMM_OK : GEMM_ERR_UNSUPPORTED_DEVICE;
}

// ---------------------------------------------------------------------------
// Argument checks (no HIP calls).
bool overlaps(const void *p, size_t pb, const void *q, size_t qb) {
  if (!pb || !qb) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), a1 = a0 + pb;
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(q), b1 = b0 + qb;
  return a0 < b1 && b0 < a1;
}

int validate(const float *A, const float *B, const float *C, int M, int N, int K) {
  if (M < 0 || N < 0 || K < 0) return GEMM_ERR_INVALID_DIM;
  // Tile and workgroup counts are kept in int on the device.
  if ((long long)M * N > (1LL << 40) || (long long)M * K > (1LL << 40) ||
      (long long)K * N > (1LL << 40))
    return GEMM_ERR_INVALID_DIM;
  // An operand is touched only when there is an output to produce (M, N > 0),
  // and A and B only when the sum is not empty (K > 0).
  const bool any_out = M > 0 && N > 0;
  const size_t a_bytes = any_out ? sizeof(float) * (size_t)M * (size_t)K : 0;
  const size_t b_bytes = any_out ? sizeof(float) * (size_t)K * (size_t)N : 0;
  const size_t c_bytes = any_out ? sizeof(float) * (size_t)M * (size_t)N : 0;
  if ((a_bytes && !A) || (b_bytes && !B) || (c_bytes && !C)) return GEMM_ERR_NULL_PTR;
  if (overlaps(C, c_bytes, A, a_bytes) || overlaps(C, c_bytes, B, b_bytes)) return GEMM_ERR_ALIAS;
  return GEMM_OK;
}

// ---------------------------------------------------------------------------
// Launch helpers.
template <int MI, int BM, int BN, int BK, int WAVES_M, int WAVES_N, int WPE, int VA, int VB,
          bool CHECK>
void launch_mfma_t(const float *A, const float *B, float *out, int M, int N, int K,
                   const Resolved &r, long long slab, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(r.tiles_m * r.tiles_n * r.splits));
  hipLaunchKernelGGL(
      (gemm::mfma_gemm_kernel<MI, BM, BN, BK, WAVES_M, WAVES_N, VA, VB, CHECK, WPE>), grid,
      dim3(64 * WAVES_M * WAVES_N), 0, stream, A, B, out, M, N, K, r.k_chunk,
      static_cast<int>(r.tiles_m), static_cast<int>(r.tiles_n), r.splits, slab);
}

bool aligned16(const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// Picks the load width and edge-check variant of one tile configuration.
// WPE = waves per SIMD the register allocation is sized for. Configurations
// with SCALAR = false have no 4-byte-load variants (they would not fit their
// register budget): they return false for shapes that need them.
template <int MI, int BM, int BN, int BK, int WAVES_M, int WAVES_N, int WPE, bool SCALAR>
bool launch_mfma(const float *A, const float *B, float *out, int M, int N, int K,
                 const Resolved &r, long long slab, hipStream_t stream) {
  const bool va = (K % 4 == 0) && aligned16(A);
  const bool vb = (N % 4 == 0) && aligned16(B);
  const bool exact = (M % BM == 0) && (N % BN == 0) && (K % BK == 0) && (r.k_chunk % BK == 0);
#define LGEMM_CASE(VA_, VB_, CK_)                                                             \
  launch_mfma_t<MI, BM, BN, BK, WAVES_M, WAVES_N, WPE, VA_, VB_, CK_>(A, B, out, M, N, K, r, \
                                                                     slab, stream)
  if (va && vb) {
    if (exact) LGEMM_CASE(4, 4, false); else LGEMM_CASE(4, 4, true);
    return true;
  }
  if constexpr (SCALAR) {
    if (va) LGEMM_CASE(4, 1, true);
    else if (vb) LGEMM_CASE(1, 4, true);
    else LGEMM_CASE(1, 1, true);
    return true;
  }
#undef LGEMM_CASE
  return false;
}

// Kernels fed by direct global -> LDS copies (16-byte copies from 4-byte
// aligned sources, any K and N). Each lane's byte offset from its tile's
// first element (at most BM*K*4 for A, (k_chunk+BK)*N*4 for B) must stay
// below 2^31; returns false (nothing launched) for shapes outside that.
template <int MI, int BM, int BN, int BK, int WAVES_M, int WAVES_N, int NS, int WPE>
bool launch_dma(const float *A, const float *B, float *out, int M, int N, int K,
                const Resolved &r, long long slab, hipStream_t stream) {
  if ((long long)BM * K * 4 >= (1LL << 31) ||
      ((long long)r.k_chunk + BK) * N * 4 >= (1LL << 31))
    return false;
  const dim3 grid(static_cast<unsigned>(r.tiles_m * r.tiles_n * r.splits));
  hipLaunchKernelGGL((gemm::mfma_dma_gemm_kernel<MI, BM, BN, BK, WAVES_M, WAVES_N, NS, 4, WPE>),
                     grid, dim3(64 * WAVES_M * WAVES_N), 0, stream, A, B, out, M, N, K,
                     r.k_chunk, static_cast<int>(r.tiles_m), static_cast<int>(r.tiles_n),
                     r.splits, slab);
  return true;
}

// Launch the kernel of r.k (falling back to a configuration with 4-byte
// loads where the chosen one has none for this shape).
void launch_gemm_kernel(const float *A, const float *B, float *out, int M, int N, int K,
                        const Resolved &r, long long slab, hipStream_t stream) {
  switch (r.k->id) {
    case GEMM_KERNEL_MFMA_256x256:
      launch_mfma<32, 256, 256, 16, 2, 2, 1, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_MFMA_256x256_W8:
      if (!launch_mfma<32, 256, 256, 16, 2, 4, 2, false>(A, B, out, M, N, K, r, slab, stream))
        launch_mfma<32, 256, 256, 16, 2, 2, 1, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_MFMA_256x128:
      launch_mfma<32, 256, 128, 16, 2, 2, 1, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_MFMA_128x128:
      launch_mfma<32, 128, 128, 16, 2, 2, 2, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_MFMA_64x64:
      launch_mfma<32, 64, 64, 16, 2, 2, 2, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_MFMA16_256x256:
      launch_mfma<16, 256, 256, 32, 2, 2, 1, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_MFMA16_256x256_W8:
      if (!launch_mfma<16, 256, 256, 32, 2, 4, 2, false>(A, B, out, M, N, K, r, slab, stream))
        launch_mfma<16, 256, 256, 32, 2, 2, 1, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_MFMA16_256x128:
      launch_mfma<16, 256, 128, 32, 2, 2, 1, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_MFMA16_128x128:
      launch_mfma<16, 128, 128, 32, 2, 2, 2, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_MFMA16_64x64:
      launch_mfma<16, 64, 64, 32, 2, 2, 2, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_MFMA16_256x256_K16:
      launch_mfma<16, 256, 256, 16, 2, 2, 1, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_MFMA16_128x128_K16:
      launch_mfma<16, 128, 128, 16, 2, 2, 2, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_MFMA16_256x128_K16:
      launch_mfma<16, 256, 128, 16, 2, 2, 1, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_MFMA_128x128_W1:
      launch_mfma<32, 128, 128, 16, 1, 1, 1, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_MFMA16_128x128_W1:
      launch_mfma<16, 128, 128, 16, 1, 1, 1, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_MFMA_64x64_W1:
      launch_mfma<32, 64, 64, 16, 1, 1, 2, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_DMA32_256x256_W8:
      if (!launch_dma<32, 256, 256, 16, 2, 4, 4, 2>(A, B, out, M, N, K, r, slab, stream))
        launch_mfma<32, 256, 256, 16, 2, 2, 1, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_DMA32_256x256_W8_S3:
      if (!launch_dma<32, 256, 256, 16, 2, 4, 3, 2>(A, B, out, M, N, K, r, slab, stream))
        launch_mfma<32, 256, 256, 16, 2, 2, 1, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_DMA16_256x256_W8:
      if (!launch_dma<16, 256, 256, 16, 2, 4, 4, 2>(A, B, out, M, N, K, r, slab, stream))
        launch_mfma<32, 256, 256, 16, 2, 2, 1, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_DMA32_128x128_W4:
      if (!launch_dma<32, 128, 128, 16, 2, 2, 4, 2>(A, B, out, M, N, K, r, slab, stream))
        launch_mfma<32, 128, 128, 16, 2, 2, 2, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_DMA16_128x128_W4:
      if (!launch_dma<16, 128, 128, 16, 2, 2, 4, 2>(A, B, out, M, N, K, r, slab, stream))
        launch_mfma<32, 128, 128, 16, 2, 2, 2, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_DMA16_64x64:
      launch_dma<16, 64, 64, 32, 2, 2, 4, 2>(A, B, out, M, N, K, r, slab, stream) ||
          launch_mfma<16, 64, 64, 32, 2, 2, 2, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_DMA32_64x64:
      launch_dma<32, 64, 64, 16, 2, 2, 4, 2>(A, B, out, M, N, K, r, slab, stream) ||
          launch_mfma<32, 64, 64, 16, 2, 2, 2, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_DMA16_128x64:
      launch_dma<16, 128, 64, 32, 2, 2, 4, 2>(A, B, out, M, N, K, r, slab, stream) ||
          launch_mfma<16, 64, 64, 32, 2, 2, 2, true>(A, B, out, M, N, K, r, slab, stream);
      return;
    case GEMM_KERNEL_VALU_64x64: {
      const bool exact = (M % 64 == 0) && (N % 64 == 0) && (K % 16 == 0);
      const dim3 grid(static_cast<unsigned>(r.tiles_m * r.tiles_n * r.splits));
      if (exact)
        hipLaunchKernelGGL(gemm::valu_gemm_kernel<false>, grid, dim3(gemm::kThreads), 0, stream, A,
                           B, out, M, N, K, r.k_chunk, (int)r.tiles_m, (int)r.tiles_n, r.splits, slab);
      else
        hipLaunchKernelGGL(gemm::valu_gemm_kernel<true>, grid, dim3(gemm::kThreads), 0, stream, A,
                           B, out, M, N, K, r.k_chunk, (int)r.tiles_m, (int)r.tiles_n, r.splits, slab);
      return;
    }
    case GEMM_KERNEL_LADDER_V0:
    case GEMM_KERNEL_LADDER_V1:
    case GEMM_KERNEL_LADDER_V2:
    case GEMM_KERNEL_LADDER_V3: {
      const dim3 grid(static_cast<unsigned>(r.tiles_m * r.tiles_n * r.splits));
      auto *kern = r.k->id == GEMM_KERNEL_LADDER_V0   ? gemm::ladder_naive_kernel<true>
                   : r.k->id == GEMM_KERNEL_LADDER_V1 ? gemm::ladder_naive_kernel<false>
                   : r.k->id == GEMM_KERNEL_LADDER_V2 ? gemm::ladder_lds_kernel
                                                      : gemm::ladder_coarse_kernel;
      hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, A, B, out, M, N, K, r.k_chunk,
                         (int)r.tiles_m, (int)r.tiles_n, r.splits, slab);
      return;
    }
  }
}

int launch(const float *A, const float *B, float *C, int M, int N, int K, const Resolved &r,
           void *workspace, hipStream_t stream) {
  float *out = r.splits > 1 ? static_cast<float *>(workspace) : C;
  const long long slab = r.splits > 1 ? (long long)M * N : 0;
  launch_gemm_kernel(A, B, out, M, N, K, r, slab, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  if (r.splits > 1) {
    const long long count = (long long)M * N;
    const bool v4 = (count % 4 == 0) && (reinterpret_cast<uintptr_t>(C) % 16 == 0) &&
                    (reinterpret_cast<uintptr_t>(workspace) % 16 == 0);
    const long long items = v4 ? count / 4 : count;
    const unsigned blocks =
        static_cast<unsigned>(std::min<long long>(ceil_div(items, gemm::kThreads), 4 * kNumCus));
    if (v4)
      hipLaunchKernelGGL(gemm::splitk_reduce_kernel<4>, dim3(blocks), dim3(gemm::kThreads), 0,
                         stream, static_cast<const float *>(workspace), C, count, r.splits);
    else
      hipLaunchKernelGGL(gemm::splitk_reduce_kernel<1>, dim3(blocks), dim3(gemm::kThreads), 0,
                         stream, static_cast<const float *>(workspace), C, count, r.splits);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e);
  }
  return GEMM_OK;
}

int launch_fill_zero(float *C, long long count, hipStream_t stream) {
  const unsigned blocks =
      static_cast<unsigned>(std::min<long long>(ceil_div(count, gemm::kThreads), 4 * kNumCus));
  hipLaunchKernelGGL(gemm::fill_zero_kernel, dim3(blocks), dim3(gemm::kThreads), 0, stream, C,
                     count);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? GEMM_OK : hip_fail(e);
}

// Common path for every entry point. `plan_in` null = planner. `own_ws`:
// use (and grow) the library's per-device workspace instead of the caller's.
int run(const float *A, const float *B, float *C, int M, int N, int K, const gemm_plan_t *plan_in,
        void *workspace, size_t workspace_bytes, bool own_ws, hipStream_t stream) {
  int st = validate(A, B, C, M, N, K);
  if (st != GEMM_OK) return st;
  int kernel = GEMM_KERNEL_AUTO, split = 1;
  if (plan_in) {
    kernel = plan_in->kernel;
    split = plan_in->split_k;
    if (kernel != GEMM_KERNEL_AUTO && (!find_kernel(kernel) || split < 1))
      return GEMM_ERR_INVALID_PLAN;
  }
  if (kernel == GEMM_KERNEL_AUTO) plan(M, N, K, &kernel, &split);
  Resolved r;
  if (!resolve(M, N, K, kernel, split, &r)) return GEMM_ERR_INVALID_PLAN;
  const size_t need = workspace_for(M, N, r);
  if (!own_ws && need > 0 && (workspace == nullptr || workspace_bytes < need))
    return GEMM_ERR_WORKSPACE;
  if (M == 0 || N == 0) return GEMM_OK;

  int dev = 0;
  st = check_device(&dev);
  if (st != GEMM_OK) return st;
  if (K == 0) return launch_fill_zero(C, (long long)M * N, stream);

  if (own_ws && need > 0) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ws_bytes[dev] < need) {
      if (g_ws[dev]) {
        hipError_t e = hipDeviceSynchronize();
        if (e != hipSuccess) return hip_fail(e);
        (void)hipFree(g_ws[dev]);
        g_ws[dev] = nullptr;
        g_ws_bytes[dev] = 0;
      }
      void *p = nullptr;
      if (hipMalloc(&p, need) == hipSuccess) {
        g_ws[dev] = p;
        g_ws_bytes[dev] = need;
      } else {
        (void)hipGetLastError();
      }
    }
    if (g_ws_bytes[dev] >= need) {
      workspace = g_ws[dev];
    } else {
      // No workspace available: same kernel without the split.
      if (!resolve(M, N, K, kernel, 1, &r)) return GEMM_ERR_INVALID_PLAN;
      workspace = nullptr;
    }
  }
  return launch(A, B, C, M, N, K, r, workspace, stream);
}

}  // namespace

extern "C" {

int gemm_f32(const float *A, const float *B, float *C, int M, int N, int K, hipStream_t stream) {
  return run(A, B, C, M, N, K, nullptr, nullptr, 0, true, stream);
}

size_t gemm_f32_workspace_bytes(int M, int N, int K) {
  if (M < 0 || N < 0 || K < 0) return 0;
  int kernel, split;
  plan(M, N, K, &kernel, &split);
  Resolved r;
  if (!resolve(M, N, K, kernel, split, &r)) return 0;
  return workspace_for(M, N, r);
}

int gemm_f32_ex(const float *A, const float *B, float *C, int M, int N, int K, void *workspace,
                size_t workspace_bytes, hipStream_t stream) {
  return run(A, B, C, M, N, K, nullptr, workspace, workspace_bytes, false, stream);
}

int gemm_f32_plan(int M, int N, int K, gemm_plan_t *out) {
  if (!out) return GEMM_ERR_NULL_PTR;
  if (M < 0 || N < 0 || K < 0) return GEMM_ERR_INVALID_DIM;
  int kernel, split;
  plan(M, N, K, &kernel, &split);
  Resolved r;
  if (!resolve(M, N, K, kernel, split, &r)) return GEMM_ERR_INVALID_PLAN;
  out->kernel = kernel;
  out->split_k = r.splits;
  out->k_chunk = r.k_chunk;
  out->reserved = 0;
  return GEMM_OK;
}

size_t gemm_f32_plan_workspace_bytes(int M, int N, int K, const gemm_plan_t *p) {
  if (!p || M < 0 || N < 0 || K < 0) return 0;
  int kernel = p->kernel, split = p->split_k;
  if (kernel == GEMM_KERNEL_AUTO) plan(M, N, K, &kernel, &split);
  Resolved r;
  if (!resolve(M, N, K, kernel, split, &r)) return 0;
  return workspace_for(M, N, r);
}

int gemm_f32_with_plan(const float *A, const float *B, float *C, int M, int N, int K,
                       const gemm_plan_t *p, void *workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  if (!p) return GEMM_ERR_INVALID_PLAN;
  return run(A, B, C, M, N, K, p, workspace, workspace_bytes, false, stream);
}

const char *gemm_kernel_name(int kernel) {
  if (kernel == GEMM_KERNEL_AUTO) return "auto";
  const KernelInfo *k = find_kernel(kernel);
  return k ? k->name : "unknown";
}

const char *gemm_status_string(int status) {
  switch (status) {
    case GEMM_OK: return "ok";
    case GEMM_ERR_INVALID_DIM: return "invalid dimension (negative or too large)";
    case GEMM_ERR_NULL_PTR: return "null pointer with nonzero extent";
    case GEMM_ERR_ALIAS: return "C overlaps A or B";
    case GEMM_ERR_WORKSPACE: return "workspace missing or too small";
    case GEMM_ERR_INVALID_PLAN: return "invalid plan (unknown kernel or split < 1)";
    case GEMM_ERR_HIP: return "HIP runtime error";
    case GEMM_ERR_UNSUPPORTED_DEVICE: return "current device is not gfx950";
    default: return "unknown status";
  }
}

int gemm_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"

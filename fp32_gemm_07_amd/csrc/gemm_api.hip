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

#include "dma_launch.hpp"
#include "gemm_kernels.hpp"
#include "ladder_kernels.hpp"

// The split-K partial sums of gemm_f32_noalloc: a static device array of
// kScratchBytes, one copy per device, allocated by the runtime when it loads
// this code object on the device and held until the process ends. On the
// host the name `scratch` is only a stand-in for it, not a device address:
// host code takes each device's address from device_scratch() and passes
// that to the kernels, never `scratch` itself.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return GEMM_ERR_HIP;
}

// Compute units assumed when no device can be queried (MI355X: 256). Plans
// for a launch use the device's own count (multiProcessorCount).
constexpr int kDefaultCus = 256;

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
    {GEMM_KERNEL_MFMA16_256x128, 256, 128, 32, "mfma16_f32_256x128x32"},
    {GEMM_KERNEL_MFMA16_128x128, 128, 128, 32, "mfma16_f32_128x128x32"},
    {GEMM_KERNEL_MFMA16_64x64, 64, 64, 32, "mfma16_f32_64x64x32"},
    {GEMM_KERNEL_MFMA16_128x128_K16, 128, 128, 16, "mfma16_f32_128x128x16"},
    {GEMM_KERNEL_MFMA16_256x128_K16, 256, 128, 16, "mfma16_f32_256x128x16"},
    {GEMM_KERNEL_MFMA_128x128_W1, 128, 128, 16, "mfma32_f32_128x128x16_w1"},
    {GEMM_KERNEL_MFMA_64x64_W1, 64, 64, 16, "mfma32_f32_64x64x16_w1"},
    {GEMM_KERNEL_VALU_64x64, 64, 64, 16, "valu_f32_64x64x16"},
    {GEMM_KERNEL_DMA32_256x256_W8, 256, 256, 16, "dma_mfma32_f32_256x256x16_w8_s4"},
    {GEMM_KERNEL_DMA32_128x128_W4, 128, 128, 16, "dma_mfma32_f32_128x128x16_w4_s4"},
    {GEMM_KERNEL_DMA16_128x128_W4, 128, 128, 16, "dma_mfma16_f32_128x128x16_w4_s4"},
    {GEMM_KERNEL_DMA32_256x256_W8_S3, 256, 256, 16, "dma_mfma32_f32_256x256x16_w8_s3"},
    {GEMM_KERNEL_DMA16_64x64, 64, 64, 32, "dma_mfma16_f32_64x64x32_w4_s4"},
    {GEMM_KERNEL_DMA32_64x64, 64, 64, 16, "dma_mfma32_f32_64x64x16_w4_s4"},
    {GEMM_KERNEL_DMA16_128x64, 128, 64, 32, "dma_mfma16_f32_128x64x32_w4_s4"},
    {GEMM_KERNEL_DMA32_128x128_W8, 128, 128, 16, "dma_mfma32_f32_128x128x16_w8_s4"},
    {GEMM_KERNEL_DMA32_64x64_S3, 64, 64, 16, "dma_mfma32_f32_64x64x16_w4_s3"},
    {GEMM_KERNEL_DMA32_128x128_W8_S3, 128, 128, 16, "dma_mfma32_f32_128x128x16_w8_s3"},
    {GEMM_KERNEL_DMA16_96x96_S3, 96, 96, 32, "dma_mfma16_f32_96x96x32_w4_s3"},
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

// The kernels fed by direct global -> LDS copies (the only ones that take a
// split tail).
bool is_dma_kernel(int id) {
  return (id >= GEMM_KERNEL_DMA32_256x256_W8 && id <= GEMM_KERNEL_DMA32_128x128_W8) ||
         id == GEMM_KERNEL_DMA32_64x64_S3 || id == GEMM_KERNEL_DMA32_128x128_W8_S3 ||
         id == GEMM_KERNEL_DMA16_96x96_S3;
}

struct Resolved {
  const KernelInfo *k;
  int splits;     // number of K ranges of a split tile (>= 1)
  int k_chunk;    // length of each K range
  long long tiles_m, tiles_n;
  long long dp_tiles;   // tiles computed whole before the split ones (split tail), else 0
  int K;
  // K elements one workgroup covers at most (its copy offsets grow with it).
  long long k_span() const { return dp_tiles > 0 ? K : k_chunk; }
  long long workgroups() const { return dp_tiles + (tiles_m * tiles_n - dp_tiles) * splits; }
};

// Turn (kernel, requested split, split tail) into launch geometry. The split
// is clamped to the number of K steps; every range then holds at least one
// element. A split tail keeps the tiles of whole rounds of `cus` tiles (one
// per compute unit) unsplit (with a whole number of rounds nothing is split).
bool resolve(int M, int N, int K, int kernel, int split_req, bool split_tail, int cus,
             Resolved *out) {
  const KernelInfo *k = find_kernel(kernel);
  if (!k || split_req < 1) return false;
  if (split_tail && !is_dma_kernel(kernel)) return false;
  out->k = k;
  out->tiles_m = ceil_div(M, k->bm);
  out->tiles_n = ceil_div(N, k->bn);
  out->dp_tiles = 0;
  out->K = K;
  const long long ksteps = std::max<long long>(1, ceil_div(K, k->bk));
  const long long s = std::min<long long>(split_req, ksteps);
  const long long chunk = ceil_div(ceil_div(std::max(K, 1), s), k->bk) * k->bk;
  out->k_chunk = static_cast<int>(std::min<long long>(chunk, INT_MAX));
  out->splits = static_cast<int>(K > 0 ? ceil_div(K, out->k_chunk) : 1);
  if (split_tail && out->splits > 1) {
    const long long tiles = out->tiles_m * out->tiles_n;
    const long long dp = tiles / cus * cus;
    if (dp == tiles) return resolve(M, N, K, kernel, 1, false, cus, out);
    out->dp_tiles = dp;
  }
  // Workgroup ids and tile indices are ints on the device.
  return out->workgroups() <= INT_MAX;
}

// The tile order of a launch, its divisors prepared for the device.
gemm::TileOrder tile_order(const Resolved &r) {
  return gemm::make_tile_order(static_cast<int>(r.tiles_m), static_cast<int>(r.tiles_n), r.splits,
                               static_cast<int>(r.dp_tiles));
}

size_t workspace_for(int M, int N, const Resolved &r) {
  return r.splits > 1 ? sizeof(float) * (size_t)r.splits * (size_t)M * (size_t)N : 0;
}

// One product C <- alpha * op(A) op(B) + beta * C on strided row-major
// storage (the plain entry points: no transposes, lda = K, ldb = N, ldc = N,
// alpha = 1, beta = 0).
struct Problem {
  bool ta, tb;   // op(A) = A^T (A stored K x M), op(B) = B^T (B stored N x K)
  int M, N, K;
  float alpha, beta;
  const float *A, *B;
  float *C;
  int lda, ldb, ldc;
};

Problem plain_problem(const float *A, const float *B, float *C, int M, int N, int K) {
  return Problem{false, false, M, N, K, 1.0f, 0.0f, A, B, C, K, N, N};
}

// The copy-fed kernels address an operand tile with 32-bit byte offsets from
// its first element: they must stay below 2^31 over the K range of one
// workgroup. K-contiguous operand: about (BX*ld + k_span)*4 bytes;
// M/N-contiguous: about (k_span*ld + BX)*4.
// Counted in floats (bx <= 256, ld and k_span below 2^32: no overflow in
// 64 bits), compared with 2^31 bytes / 4.
constexpr long long kMaxOffsetFloats = (1LL << 31) / 4;
bool operand_fits(bool kmajor, int bx, int ld, long long k_span) {
  const long long floats = kmajor ? (long long)bx * ld + k_span : k_span * ld + bx;
  return floats < kMaxOffsetFloats;
}
bool dma_fits(const Problem &p, int bm, int bn, int bk, int k_chunk) {
  const long long span = (long long)k_chunk + bk;
  return operand_fits(!p.ta, bm, p.lda, span) && operand_fits(p.tb, bn, p.ldb, span);
}
// The K-contiguous limit does not depend on K: whether a tile size can be
// used at all for these row strides.
bool dma_tile_usable(const Problem &p, int bm, int bn, int bk) {
  return (p.ta || operand_fits(true, bm, p.lda, 2 * bk)) &&
         (!p.tb || operand_fits(true, bn, p.ldb, 2 * bk));
}

// The planner: a cost model over five copy-fed kernels and power-of-two
// K splits, fitted to timings of those kernels over square, wide, long-K and
// ragged shapes on one MI355X. A CU works through its share of a launch's
// workgroups (at most n = ceil(workgroups / CUs) of them), so a launch costs
//   n * (2 * BM * BN * k_chunk / (rate_cu * eff) + per_wg) + fixed
// with rate_cu = 256 FLOP/clk at 2.38 GHz and eff, per_wg (prologue and
// epilogue of one workgroup) and fixed (launch, clock skew between XCDs)
// per kernel below. With a split tail each CU takes dp_tiles / CUs whole
// tiles, then its share of the split ones. Splitting K adds the partial sums
// of the split tiles (S slabs written and read, C written), which stay in
// the last-level cache at these sizes, at about 8 TB/s plus a fixed cost for
// the extra launch; and no launch is cheaper than moving A, B and C once at
// about 5 TB/s. Workspace is capped at 1 GiB.
struct PlanCandidate {
  int kernel;
  double eff;
  double per_wg_us;
  double fixed_us;
  int slots_per_cu;           // workgroups one CU holds at once (two waves per SIMD)
  double eff_shared;          // eff when the launch puts more than one workgroup on a CU
  double per_wg_shared_us;    // per_wg then (one workgroup's store overlaps another's work)
  bool all_orders;            // built for transposed operands too
  bool paired_tail;           // split tail: pieces may land two to a CU (see plan_cost_us)
  int min_k;                  // not considered for shorter K
};
// With two 64x64 workgroups on a CU each SIMD runs two waves, which hide
// each other's waits: per-wave timestamps give 1,083 clocks per pair of K
// steps against 1,024 of MFMA (0.945), one workgroup alone 0.91. The 4-wave
// 128x128 kernel, last, is for short K over large outputs, where the store
// of C bounds the launch and two workgroups per CU overlap one's store with
// the other's copies (8192 x 16 x 8192: 52.7 against 62.1 us for 256x256);
// from K ~ 128 (4096^2) or ~ 200 (8192^2) on it loses to the others
// (4096 x 256 x 4096: 77.2 against 73.1 us), which its eff_shared is fitted to.
// The 96 x 96 kernel (16 x 16 blocks, one wave per SIMD) fills the CUs where
// 64 x 64 and 128 x 128 tiles leave a partial round: 256 tiles at 1536^2
// (54.8 against 61.3 us for the best 64 x 64 plan), 1024 at 3072^2. Its
// constants are fitted to 59 shapes (square, wide, long-K, short-K, small
// and ragged) timed with all five candidates: the planner's plan is within
// 2 % of the fastest candidate plan on 55 of them (on 43 without this
// kernel). Its low eff stands for the dearer prologue of short K ranges
// (333 x 4444 x 555 split in 8: 31.2 against 25.0 us for 64 x 64 tiles). It
// comes last, so that it takes only plans more than 1 % cheaper than the
// others' (ties go to the plan seen first), and only from K = 64 (two of its
// K steps): below that the fill of its three 24 KiB stages is most of a
// launch that the model's other candidates are costed too dearly for
// (2048 x 16 x 2048: 10.1 us against 9.0 for 128 x 128 tiles).
constexpr PlanCandidate kPlanCandidates[] = {
    {GEMM_KERNEL_DMA32_256x256_W8_S3, 0.966, 11.9, 5.6, 1, 0.966, 11.9, true, false, 0},
    {GEMM_KERNEL_DMA32_128x128_W8_S3, 0.982, 6.9, 3.9, 1, 0.982, 6.9, true, false, 0},
    {GEMM_KERNEL_DMA32_64x64_S3, 0.91, 1.2, 6.5, 2, 0.935, 1.2, true, true, 0},
    {GEMM_KERNEL_DMA32_128x128_W4, 0.95, 7.0, 3.9, 2, 0.86, 2.0, true, true, 0},
    {GEMM_KERNEL_DMA16_96x96_S3, 0.95, 2.0, 4.0, 2, 0.97, 2.0, true, false, 64},
};
constexpr double kRateCuFlopPerUs = 256.0 * 2.38e3;   // FLOP per microsecond per CU
constexpr double kReduceBytesPerUs = 8.0e6;           // split-K partial sums
constexpr double kReduceFixedUs = 2.0;
constexpr double kMaxWorkspaceBytes = 1024.0 * 1024.0 * 1024.0;
constexpr double kHbmBytesPerUs = 5.0e6;

// A (kernel, split) whose copy offsets would not fit in 32 bits is not
// considered (the launch would fall back to a slower kernel or K passes).
// *r_out: the geometry costed.
double plan_cost_us(const Problem &pr, const PlanCandidate &c, int split, bool tail, int cus,
                    Resolved *r_out) {
  const int M = pr.M, N = pr.N, K = pr.K;
  Resolved &r = *r_out;
  if (!resolve(M, N, K, c.kernel, split, tail, cus, &r)) return 1e30;
  if (!dma_fits(pr, r.k->bm, r.k->bn, r.k->bk, r.k_span())) return 1e30;
  const double tile_flop = 2.0 * r.k->bm * r.k->bn;
  const double split_tiles = static_cast<double>(r.tiles_m * r.tiles_n - r.dp_tiles);
  const bool shared = static_cast<double>(r.workgroups()) > cus;
  const double eff = shared ? c.eff_shared : c.eff;
  const double per_wg_us = shared ? c.per_wg_shared_us : c.per_wg_us;
  const double per_wg = tile_flop * r.k_chunk / (kRateCuFlopPerUs * eff) + per_wg_us;
  double rounds = std::ceil(split_tiles * r.splits / cus);
  // The pieces of a split tail start as the whole tiles end, on whichever CU
  // frees a slot first. A CU holds two workgroups of a 4-wave kernel: with
  // more pieces than half the CUs some CU can take two of them side by side,
  // so such a round is costed as two (paired_tail). How much that costs
  // depends on how the whole tiles end: 256 pieces of 64 x 64 tiles after two
  // whole rounds take 66 against 62 us for 128 pieces at 1500^3 (the rule's
  // choice), but 61 against 63.5 us at 1536^3, where the rule picks the 128
  // (three runs each); without the rule the two swap, with no gain over the
  // shapes measured. The 96 x 96 kernel's tails follow the plain rounds
  // (2304^3: 256 pieces 177.1, 512 pieces 183.7 us; 1792^3: 210 pieces 95.3,
  // 420 pieces 99.9 us).
  if (r.dp_tiles > 0 && c.paired_tail && split_tiles * r.splits > cus / 2)
    rounds = std::max(rounds, 2.0);
  double us = rounds * per_wg + c.fixed_us;
  if (r.dp_tiles > 0)
    us += static_cast<double>(r.dp_tiles / cus) *
          (tile_flop * static_cast<double>(r.k_span()) / (kRateCuFlopPerUs * eff) + per_wg_us);
  if (r.splits > 1) {
    const double slab = 4.0 * M * static_cast<double>(N);
    if (slab * r.splits > kMaxWorkspaceBytes) return 1e30;
    const double split_bytes =
        r.dp_tiles > 0 ? 4.0 * split_tiles * r.k->bm * r.k->bn : slab;
    us += (2.0 * r.splits + 1.0) * split_bytes / kReduceBytesPerUs + kReduceFixedUs;
  }
  // No launch beats reading A and B and writing C once (about 5 TB/s).
  const double bytes = 4.0 * (static_cast<double>(M) * K + static_cast<double>(K) * N +
                              static_cast<double>(M) * N);
  return std::max(us, bytes / kHbmBytesPerUs + c.fixed_us);
}

struct PlanChoice {
  int kernel;
  int split;
  bool tail;   // split only the last, partial round of tiles
};

PlanChoice plan(int M, int N, int K, int cus, const Problem *general = nullptr) {
  PlanChoice best_plan{kPlanCandidates[0].kernel, 1, false};
  double best = 1e30;
  Problem pr = general ? *general : plain_problem(nullptr, nullptr, nullptr, M, N, K);
  pr.K = K;
  for (const PlanCandidate &c : kPlanCandidates) {
    if (K < c.min_k) continue;
    if (general) {
      const KernelInfo *k = find_kernel(c.kernel);
      if (!c.all_orders && (general->ta || general->tb)) continue;
      if (!dma_tile_usable(*general, k->bm, k->bn, k->bk)) continue;
    }
    for (int s = 1; s <= 64; s *= 2) {
      if (s > 1 && K / s < 256) break;   // each K range keeps >= 256 elements
      for (int tail = 0; tail <= (s > 1 ? 1 : 0); ++tail) {
        Resolved r;
        const double us = plan_cost_us(pr, c, s, tail != 0, cus, &r);
        if (us >= 1e30) continue;
        if (r.splits < s) break;                // fewer K steps than ranges asked for
        if (tail && r.dp_tiles == 0) continue;  // the same as splitting every tile
        // Ties (within 1%) go to the plan seen first: bigger tiles, fewer
        // splits, every tile split before a split tail.
        if (us < best * 0.99) {
          best = us;
          best_plan = PlanChoice{c.kernel, s, tail != 0};
        }
      }
    }
  }
  return best_plan;
}

// ---------------------------------------------------------------------------
// Per-device state, filled on first use of a device under g_mu: whether it is
// gfx950 (the code objects are built for gfx950 only) and its compute-unit
// count (the planner's rounds of tiles).
std::mutex g_mu;
constexpr int kMaxDevices = 64;
struct DeviceState {
  int arch;          // 0 not queried yet, 1 gfx950, -1 another architecture
  int cus;           // multiProcessorCount
  float *scratch;    // this device's copy of `scratch` (null until first looked up)
};
DeviceState g_dev[kMaxDevices];

// The current device and its compute units (properties read once per device).
hipError_t current_device(int *dev_out, int *cus_out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState &d = g_dev[dev];
  if (d.arch == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return e;
    d.cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : kDefaultCus;
    d.arch = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
  }
  *dev_out = dev;
  *cus_out = d.cus;
  return hipSuccess;
}

// The device a launch will run on: the current one, which must be gfx950.
int check_device(int *dev_out, int *cus_out) {
  const hipError_t e = current_device(dev_out, cus_out);
  if (e == hipErrorInvalidDevice) return GEMM_ERR_UNSUPPORTED_DEVICE;
  if (e != hipSuccess) return hip_fail(e);
  return g_dev[*dev_out].arch == 1 ? GEMM_OK : GEMM_ERR_UNSUPPORTED_DEVICE;
}

// Compute units to plan for in a query that launches nothing: the current
// device's, or kDefaultCus when no device can be queried (a host without a
// GPU). Leaves the thread's last HIP error untouched.
int planning_cus() {
  int dev = 0, cus = kDefaultCus;
  if (current_device(&dev, &cus) != hipSuccess) {
    (void)hipGetLastError();
    return kDefaultCus;
  }
  return cus;
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
// WPE = waves per SIMD the register allocation of the 16-byte-load variants
// is sized for, SWPE the same for the variants with 4-byte loads of A or B
// (four times the staging registers); SWPE = 0: no such variants (they would
// spill at any budget), and shapes that need them return false.
template <int MI, int BM, int BN, int BK, int WAVES_M, int WAVES_N, int WPE, int SWPE>
bool launch_mfma(const float *A, const float *B, float *out, int M, int N, int K,
                 const Resolved &r, long long slab, hipStream_t stream) {
  const bool va = (K % 4 == 0) && aligned16(A);
  const bool vb = (N % 4 == 0) && aligned16(B);
  const bool exact = (M % BM == 0) && (N % BN == 0) && (K % BK == 0) && (r.k_chunk % BK == 0);
#define LGEMM_CASE(W_, VA_, VB_, CK_)                                                       \
  launch_mfma_t<MI, BM, BN, BK, WAVES_M, WAVES_N, W_, VA_, VB_, CK_>(A, B, out, M, N, K, r, \
                                                                    slab, stream)
  if (va && vb) {
    if (exact) LGEMM_CASE(WPE, 4, 4, false); else LGEMM_CASE(WPE, 4, 4, true);
    return true;
  }
  if constexpr (SWPE > 0) {
    if (va) LGEMM_CASE(SWPE, 4, 1, true);
    else if (vb) LGEMM_CASE(SWPE, 1, 4, true);
    else LGEMM_CASE(SWPE, 1, 1, true);
    return true;
  }
#undef LGEMM_CASE
  return false;
}

// Kernels fed by direct global -> LDS copies (16-byte copies from 4-byte
// aligned sources, any K, N and row strides, either storage order of each
// operand), launched from their own translation unit (dma_launch.hpp).
// Whole tiles get alpha * op(A) op(B) + beta * C, split ones their K range's
// partial product in workspace slab s (ws + s * slab, row stride N). Returns
// false (nothing launched) when the operand offsets of one workgroup would
// not fit in 32 bits, or the configuration is not built for the operands'
// storage order.
bool launch_dma(const Problem &p, float *ws, const Resolved &r, long long slab,
                hipStream_t stream) {
  const KernelInfo &k = *r.k;
  if (!dma_fits(p, k.bm, k.bn, k.bk, r.k_span())) return false;
  const gemm::DmaLaunch d{p.A,     p.B,      p.C,  ws,   p.M,       p.N,  p.K,
                          p.lda,   p.ldb,    p.ldc, p.alpha, p.beta, p.ta, p.tb,
                          r.k_chunk, slab,   gemm::kernel_order(tile_order(r)), r.workgroups()};
  return gemm::launch_dma_kernel(k.id, d, stream);
}

// Launch the kernel of r.k for the product or, when r splits K, the partial
// products into the workspace (slabs of M x N). Register-staged, vector-FMA
// and ladder kernels write `out` (C, or the workspace when split) with row
// stride N and take the plain problem only (op = identity, dense operands;
// alpha = 1, beta = 0, ldc = N unless split) and no split tail; a copy-fed
// kernel whose offsets would not fit runs the register-staged kernel of its
// tile for such a problem. Returns false if nothing could be launched.
bool launch_gemm_kernel(const Problem &p, void *workspace, const Resolved &r,
                        hipStream_t stream) {
  const float *A = p.A, *B = p.B;
  const int M = p.M, N = p.N, K = p.K;
  const bool split = r.splits > 1;
  float *ws = static_cast<float *>(workspace);
  float *out = split ? ws : p.C;
  const long long slab = split ? (long long)M * N : 0;
  const bool plain = !p.ta && !p.tb && p.lda == K && p.ldb == N && r.dp_tiles == 0 &&
                     (split || (p.ldc == N && p.alpha == 1.0f && p.beta == 0.0f));
  const bool dma_kernel = is_dma_kernel(r.k->id);
  if (!plain && !dma_kernel) return false;
  switch (r.k->id) {
    case GEMM_KERNEL_MFMA_256x256:
      launch_mfma<32, 256, 256, 16, 2, 2, 1, 1>(A, B, out, M, N, K, r, slab, stream);
      return true;
    case GEMM_KERNEL_MFMA_256x256_W8:
      if (!launch_mfma<32, 256, 256, 16, 2, 4, 2, 0>(A, B, out, M, N, K, r, slab, stream))
        launch_mfma<32, 256, 256, 16, 2, 2, 1, 1>(A, B, out, M, N, K, r, slab, stream);
      return true;
    case GEMM_KERNEL_MFMA_256x128:
      launch_mfma<32, 256, 128, 16, 2, 2, 1, 1>(A, B, out, M, N, K, r, slab, stream);
      return true;
    case GEMM_KERNEL_MFMA_128x128:
      launch_mfma<32, 128, 128, 16, 2, 2, 2, 2>(A, B, out, M, N, K, r, slab, stream);
      return true;
    case GEMM_KERNEL_MFMA_64x64:
      launch_mfma<32, 64, 64, 16, 2, 2, 2, 2>(A, B, out, M, N, K, r, slab, stream);
      return true;
    case GEMM_KERNEL_MFMA16_256x128:
      launch_mfma<16, 256, 128, 32, 2, 2, 1, 1>(A, B, out, M, N, K, r, slab, stream);
      return true;
    case GEMM_KERNEL_MFMA16_128x128:
      launch_mfma<16, 128, 128, 32, 2, 2, 2, 1>(A, B, out, M, N, K, r, slab, stream);
      return true;
    case GEMM_KERNEL_MFMA16_64x64:
      launch_mfma<16, 64, 64, 32, 2, 2, 2, 2>(A, B, out, M, N, K, r, slab, stream);
      return true;
    case GEMM_KERNEL_MFMA16_128x128_K16:
      launch_mfma<16, 128, 128, 16, 2, 2, 2, 2>(A, B, out, M, N, K, r, slab, stream);
      return true;
    case GEMM_KERNEL_MFMA16_256x128_K16:
      // Shapes that need 4-byte loads run the same 256 x 128 tile (the same
      // geometry) with v_mfma_f32_32x32x2_f32: with them this configuration
      // spills even at one wave per SIMD.
      if (!launch_mfma<16, 256, 128, 16, 2, 2, 1, 0>(A, B, out, M, N, K, r, slab, stream))
        launch_mfma<32, 256, 128, 16, 2, 2, 1, 1>(A, B, out, M, N, K, r, slab, stream);
      return true;
    case GEMM_KERNEL_MFMA_128x128_W1:
      launch_mfma<32, 128, 128, 16, 1, 1, 1, 1>(A, B, out, M, N, K, r, slab, stream);
      return true;
    case GEMM_KERNEL_MFMA_64x64_W1:
      launch_mfma<32, 64, 64, 16, 1, 1, 2, 2>(A, B, out, M, N, K, r, slab, stream);
      return true;
    case GEMM_KERNEL_DMA32_256x256_W8:
      return launch_dma(p, ws, r, slab, stream) ||
             (plain && launch_mfma<32, 256, 256, 16, 2, 2, 1, 1>(A, B, out, M, N, K, r, slab,
                                                                    stream));
    case GEMM_KERNEL_DMA32_256x256_W8_S3:
      return launch_dma(p, ws, r, slab, stream) ||
             (plain && launch_mfma<32, 256, 256, 16, 2, 2, 1, 1>(A, B, out, M, N, K, r, slab,
                                                                    stream));
    case GEMM_KERNEL_DMA32_128x128_W4:
      return launch_dma(p, ws, r, slab, stream) ||
             (plain && launch_mfma<32, 128, 128, 16, 2, 2, 2, 2>(A, B, out, M, N, K, r, slab,
                                                                    stream));
    case GEMM_KERNEL_DMA16_128x128_W4:
      return launch_dma(p, ws, r, slab, stream) ||
             (plain && launch_mfma<32, 128, 128, 16, 2, 2, 2, 2>(A, B, out, M, N, K, r, slab,
                                                                    stream));
    case GEMM_KERNEL_DMA16_64x64:
      return launch_dma(p, ws, r, slab, stream) ||
             (plain && launch_mfma<16, 64, 64, 32, 2, 2, 2, 2>(A, B, out, M, N, K, r, slab,
                                                                  stream));
    case GEMM_KERNEL_DMA32_64x64:
      return launch_dma(p, ws, r, slab, stream) ||
             (plain && launch_mfma<32, 64, 64, 16, 2, 2, 2, 2>(A, B, out, M, N, K, r, slab,
                                                                  stream));
    case GEMM_KERNEL_DMA16_128x64:
      return launch_dma(p, ws, r, slab, stream) ||
             (plain && launch_mfma<16, 128, 64, 32, 2, 2, 2, 2>(A, B, out, M, N, K, r, slab,
                                                                   stream));
    case GEMM_KERNEL_DMA32_128x128_W8:
      return launch_dma(p, ws, r, slab, stream) ||
             (plain && launch_mfma<32, 128, 128, 16, 2, 2, 2, 2>(A, B, out, M, N, K, r, slab,
                                                                    stream));
    case GEMM_KERNEL_DMA32_128x128_W8_S3:
      return launch_dma(p, ws, r, slab, stream) ||
             (plain && launch_mfma<32, 128, 128, 16, 2, 2, 2, 2>(A, B, out, M, N, K, r, slab,
                                                                    stream));
    case GEMM_KERNEL_DMA32_64x64_S3:
      return launch_dma(p, ws, r, slab, stream) ||
             (plain && launch_mfma<32, 64, 64, 16, 2, 2, 2, 2>(A, B, out, M, N, K, r, slab,
                                                                  stream));
    case GEMM_KERNEL_DMA16_96x96_S3:   // no register-staged kernel of this tile
      return launch_dma(p, ws, r, slab, stream);
    case GEMM_KERNEL_VALU_64x64: {
      const bool exact = (M % 64 == 0) && (N % 64 == 0) && (K % 16 == 0);
      const dim3 grid(static_cast<unsigned>(r.tiles_m * r.tiles_n * r.splits));
      if (exact)
        hipLaunchKernelGGL(gemm::valu_gemm_kernel<false>, grid, dim3(gemm::kThreads), 0, stream, A,
                           B, out, M, N, K, r.k_chunk, (int)r.tiles_m, (int)r.tiles_n, r.splits,
                           slab);
      else
        hipLaunchKernelGGL(gemm::valu_gemm_kernel<true>, grid, dim3(gemm::kThreads), 0, stream, A,
                           B, out, M, N, K, r.k_chunk, (int)r.tiles_m, (int)r.tiles_n, r.splits,
                           slab);
      return true;
    }
    case GEMM_KERNEL_LADDER_V0:
    case GEMM_KERNEL_LADDER_V1:
    case GEMM_KERNEL_LADDER_V2:
    case GEMM_KERNEL_LADDER_V3: {
      const dim3 grid(static_cast<unsigned>(r.tiles_m * r.tiles_n * r.splits));
      auto *kern = r.k->id == GEMM_KERNEL_LADDER_V0   ? gemm::ladder_naive_kernel<true>
                   : r.k->id == GEMM_KERNEL_LADDER_V1 ? gemm::ladder_naive_kernel<false>
                   : r.k->id == GEMM_KERNEL_LADDER_V2 ? gemm::ladder_lds_kernel<1>
                                                      : gemm::ladder_lds_kernel<4>;
      hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, A, B, out, M, N, K, r.k_chunk,
                         (int)r.tiles_m, (int)r.tiles_n, r.splits, slab);
      return true;
    }
  }
  return false;
}

// One pass of the product with a resolved plan: the kernel, then (split K)
// the reduction of the partial slabs into C with alpha and beta, over all of
// C or (split tail) over the split tiles only.
int launch(const Problem &p, const Resolved &r, void *workspace, int cus, hipStream_t stream) {
  if (!launch_gemm_kernel(p, workspace, r, stream)) return GEMM_ERR_INVALID_PLAN;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e);
  if (r.splits > 1) {
    const long long count = (long long)p.M * p.N;
    const bool v4 = (p.N % 4 == 0) && (p.ldc % 4 == 0) &&
                    (reinterpret_cast<uintptr_t>(p.C) % 16 == 0) &&
                    (reinterpret_cast<uintptr_t>(workspace) % 16 == 0);
    const float *ws = static_cast<const float *>(workspace);
    if (r.dp_tiles > 0) {
      const int bm = r.k->bm, bn = r.k->bn;
      const long long per_tile = (long long)bm * (v4 ? bn / 4 : bn);
      const dim3 grid(static_cast<unsigned>(r.tiles_m * r.tiles_n - r.dp_tiles),
                      static_cast<unsigned>(ceil_div(per_tile, 4 * gemm::kThreads)));
      const gemm::TileOrder order = tile_order(r);
      if (v4)
        hipLaunchKernelGGL(gemm::tail_reduce_kernel<4>, grid, dim3(gemm::kThreads), 0, stream, ws,
                           p.C, p.M, p.N, p.ldc, order, bm, bn, p.alpha, p.beta);
      else
        hipLaunchKernelGGL(gemm::tail_reduce_kernel<1>, grid, dim3(gemm::kThreads), 0, stream, ws,
                           p.C, p.M, p.N, p.ldc, order, bm, bn, p.alpha, p.beta);
      e = hipGetLastError();
      return e == hipSuccess ? GEMM_OK : hip_fail(e);
    }
    const long long items = v4 ? count / 4 : count;
    const unsigned blocks =
        static_cast<unsigned>(std::min<long long>(ceil_div(items, gemm::kThreads), 4LL * cus));
    if (v4)
      hipLaunchKernelGGL(gemm::splitk_reduce_kernel<4>, dim3(blocks), dim3(gemm::kThreads), 0,
                         stream, ws, p.C, count, p.N, p.ldc, r.splits, p.alpha, p.beta);
    else
      hipLaunchKernelGGL(gemm::splitk_reduce_kernel<1>, dim3(blocks), dim3(gemm::kThreads), 0,
                         stream, ws, p.C, count, p.N, p.ldc, r.splits, p.alpha, p.beta);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e);
  }
  return GEMM_OK;
}

// C <- beta * C (+0.0 when beta == 0): the product when K = 0 or alpha = 0.
int launch_scale_c(const Problem &p, int cus, hipStream_t stream) {
  const long long count = (long long)p.M * p.N;
  const unsigned blocks =
      static_cast<unsigned>(std::min<long long>(ceil_div(count, gemm::kThreads), 4LL * cus));
  hipLaunchKernelGGL(gemm::scale_c_kernel, dim3(blocks), dim3(gemm::kThreads), 0, stream, p.C,
                     count, p.N, p.ldc, p.beta);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? GEMM_OK : hip_fail(e);
}

// ---------------------------------------------------------------------------
// The library-owned split-K workspace of gemm_f32 and gemm_f32_general (null
// workspace argument): per device, up to kMaxWsBlocks device buffers, each
// with an event recorded on the stream of the last work that used it. A call
// holds g_ws_mu from choosing a buffer until its kernels and that event are
// enqueued, so two calls never pick a buffer at the same time, and a buffer is
// handed to new work only when nothing pending can still touch it:
//   - its event has completed, or the last user was the same stream (stream
//     order then puts the new work after the old), or
//   - otherwise the new work's stream waits for the event (hipStreamWaitEvent:
//     ordered on the device, the host does not block).
// A buffer is freed (to make room for a larger one) only once its event has
// completed, so no pending kernel can be reading or writing it. Nothing here
// synchronises the device.
std::mutex g_ws_mu;
constexpr int kMaxWsBlocks = 8;
struct WsBlock {
  void *ptr;
  size_t bytes;
  hipEvent_t done;      // recorded after the last work that used the block
  hipStream_t stream;   // that work's stream
  bool recorded;        // `done` has been recorded at least once
  bool retired;         // recording failed: never handed out again (never freed)
};
WsBlock g_ws[kMaxDevices][kMaxWsBlocks];

// Whether nothing enqueued before can still use block b when new work is
// enqueued on `stream`. hipStreamPerThread names a different stream on every
// host thread, so equal handles do not imply one stream there.
int block_free_for(const WsBlock &b, hipStream_t stream, bool *free_out) {
  *free_out = !b.recorded || (b.stream == stream && stream != hipStreamPerThread);
  if (*free_out) return GEMM_OK;
  const hipError_t q = hipEventQuery(b.done);
  if (q == hipSuccess) {
    *free_out = true;
    return GEMM_OK;
  }
  if (q == hipErrorNotReady) {
    (void)hipGetLastError();
    return GEMM_OK;
  }
  return hip_fail(q);
}

// A new block of `need` bytes in slot `b` (whose previous buffer, if any, has
// been freed). Returns false, leaving the slot empty, if allocation fails.
bool new_block(WsBlock &b, size_t need) {
  void *ptr = nullptr;
  hipEvent_t ev = nullptr;
  if (hipMalloc(&ptr, need) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(ptr);   // never used by any kernel
    return false;
  }
  b = WsBlock{ptr, need, ev, nullptr, false, false};
  return true;
}

// Picks a block of at least `need` bytes for work about to be enqueued on
// `stream` (g_ws_mu held), making the stream wait for the block's previous
// user where needed. *out = null: no block could be had (the caller then runs
// without a workspace).
int acquire_block(int dev, size_t need, hipStream_t stream, WsBlock **out) {
  *out = nullptr;
  WsBlock *slots = g_ws[dev];
  WsBlock *idle = nullptr, *busy = nullptr, *empty = nullptr, *small_idle = nullptr;
  for (int i = 0; i < kMaxWsBlocks; ++i) {
    WsBlock &b = slots[i];
    if (!b.ptr) {
      if (!empty) empty = &b;
      continue;
    }
    if (b.retired) continue;
    bool is_free = false;
    const int st = block_free_for(b, stream, &is_free);
    if (st != GEMM_OK) return st;
    if (b.bytes >= need) {
      if (is_free) {
        if (!idle || b.bytes < idle->bytes) idle = &b;
      } else if (!busy || b.bytes < busy->bytes) {
        busy = &b;
      }
    } else if (is_free && !small_idle) {
      small_idle = &b;
    }
  }
  if (idle) {
    *out = idle;
    return GEMM_OK;
  }
  // A new buffer lets this work run alongside the busy one's.
  if (empty && new_block(*empty, need)) {
    *out = empty;
    return GEMM_OK;
  }
  if (busy) {
    const hipError_t e = hipStreamWaitEvent(stream, busy->done, 0);
    if (e != hipSuccess) return hip_fail(e);
    *out = busy;
    return GEMM_OK;
  }
  // Every slot holds a smaller buffer: replace one that nothing can still use.
  if (small_idle) {
    const hipError_t e = hipFree(small_idle->ptr);
    (void)hipEventDestroy(small_idle->done);
    *small_idle = WsBlock{};
    if (e != hipSuccess) return hip_fail(e);
    if (new_block(*small_idle, need)) *out = small_idle;
  }
  return GEMM_OK;
}

// Runs body(workspace) with a library-owned workspace of at least `need` bytes
// (body(nullptr) if none could be had), then records the block's event after
// the enqueued work. Refuses a stream that is capturing a graph: the block
// bookkeeping (event queries, allocation) has no meaning inside a capture.
template <class Body>
int with_library_workspace(int dev, size_t need, hipStream_t stream, Body &&body) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) return hip_fail(e);
  if (cs != hipStreamCaptureStatusNone) return GEMM_ERR_CAPTURING;
  std::lock_guard<std::mutex> lock(g_ws_mu);
  WsBlock *b = nullptr;
  int st = acquire_block(dev, need, stream, &b);
  if (st != GEMM_OK) return st;
  if (!b) return body(nullptr);
  st = body(b->ptr);
  e = hipEventRecord(b->done, stream);
  if (e != hipSuccess) {
    // The block may still be in use and there is no event to tell when it
    // is not: keep it out of the pool for good.
    b->retired = true;
    return st != GEMM_OK ? st : hip_fail(e);
  }
  b->recorded = true;
  b->stream = stream;
  return st;
}

// This device's copy of `scratch` (the no-allocation entry point's split-K
// buffer), its address looked up once per device with that device current.
int device_scratch(int dev, float **out) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_dev[dev].scratch) {
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!ptr) return GEMM_ERR_HIP;
    g_dev[dev].scratch = static_cast<float *>(ptr);
  }
  *out = g_dev[dev].scratch;
  return GEMM_OK;
}

// Where the split-K partial sums of a plain call go.
enum class Ws {
  kCaller,    // the caller's buffer (GEMM_ERR_WORKSPACE if too small)
  kLibrary,   // the library's pool (falls back to the unsplit plan if none)
  kScratch,   // the static `scratch` array (GEMM_ERR_SCRATCH_LIMIT if too small)
};

// Common path of the plain entry points. `plan_in` null = planner.
int run(const float *A, const float *B, float *C, int M, int N, int K, const gemm_plan_t *plan_in,
        void *workspace, size_t workspace_bytes, Ws mode, hipStream_t stream) {
  int st = validate(A, B, C, M, N, K);
  if (st != GEMM_OK) return st;
  PlanChoice pc{GEMM_KERNEL_AUTO, 1, false};
  if (plan_in) {
    pc = PlanChoice{plan_in->kernel, plan_in->split_k, plan_in->split_tail != 0};
    if (pc.kernel != GEMM_KERNEL_AUTO &&
        (!find_kernel(pc.kernel) || pc.split < 1 || plan_in->split_tail < 0 ||
         plan_in->split_tail > 1))
      return GEMM_ERR_INVALID_PLAN;
  }
  const int cus = planning_cus();
  if (pc.kernel == GEMM_KERNEL_AUTO) pc = plan(M, N, K, cus);
  Resolved r;
  if (!resolve(M, N, K, pc.kernel, pc.split, pc.tail, cus, &r)) return GEMM_ERR_INVALID_PLAN;
  const size_t need = workspace_for(M, N, r);
  if (mode == Ws::kCaller && need > 0 && (workspace == nullptr || workspace_bytes < need))
    return GEMM_ERR_WORKSPACE;
  if (mode == Ws::kScratch && need > kScratchBytes) return GEMM_ERR_SCRATCH_LIMIT;
  if (M == 0 || N == 0) return GEMM_OK;

  int dev = 0, dev_cus = 0;
  st = check_device(&dev, &dev_cus);
  if (st != GEMM_OK) return st;
  const Problem p = plain_problem(A, B, C, M, N, K);
  if (mode == Ws::kScratch) {
    float *scr = nullptr;
    st = device_scratch(dev, &scr);
    if (st != GEMM_OK) return st;
    workspace = scr;
  }
  if (K == 0) return launch_scale_c(p, cus, stream);
  if (mode == Ws::kLibrary && need > 0) {
    return with_library_workspace(dev, need, stream, [&](void *ws) {
      Resolved rr = r;
      // No workspace to be had: the same kernel without the split.
      if (!ws && !resolve(M, N, K, pc.kernel, 1, false, cus, &rr)) return (int)GEMM_ERR_INVALID_PLAN;
      return launch(p, rr, ws, cus, stream);
    });
  }
  return launch(p, r, workspace, cus, stream);
}

// ---------------------------------------------------------------------------
// The general form: transposes, row strides, alpha and beta.
int validate_general(const Problem &p) {
  if (p.M < 0 || p.N < 0 || p.K < 0) return GEMM_ERR_INVALID_DIM;
  const int a_cols = p.ta ? p.M : p.K, b_cols = p.tb ? p.K : p.N;
  if (p.lda < std::max(1, a_cols) || p.ldb < std::max(1, b_cols) || p.ldc < std::max(1, p.N))
    return GEMM_ERR_INVALID_DIM;
  const long long a_rows = p.ta ? p.K : p.M, b_rows = p.tb ? p.N : p.K;
  if (a_rows * p.lda > (1LL << 40) || b_rows * p.ldb > (1LL << 40) ||
      (long long)p.M * p.ldc > (1LL << 40))
    return GEMM_ERR_INVALID_DIM;
  const bool any_out = p.M > 0 && p.N > 0;
  const bool uses_ab = any_out && p.K > 0 && p.alpha != 0.0f;
  // Byte extents from each operand's first to its last element.
  const size_t a_bytes = uses_ab ? sizeof(float) * (size_t)((a_rows - 1) * p.lda + a_cols) : 0;
  const size_t b_bytes = uses_ab ? sizeof(float) * (size_t)((b_rows - 1) * p.ldb + b_cols) : 0;
  const size_t c_bytes = any_out ? sizeof(float) * (size_t)((long long)(p.M - 1) * p.ldc + p.N) : 0;
  if ((a_bytes && !p.A) || (b_bytes && !p.B) || (c_bytes && !p.C)) return GEMM_ERR_NULL_PTR;
  if (overlaps(p.C, c_bytes, p.A, a_bytes) || overlaps(p.C, c_bytes, p.B, b_bytes))
    return GEMM_ERR_ALIAS;
  return GEMM_OK;
}

// The planner's kernel and split for the general form. Copy offsets of an
// M/N-contiguous operand grow with the K range; when one pass over all of K
// would not fit in 32 bits, K is cut into passes of *k_pass elements, run
// one after the other (the second and later with beta = 1), and the plan is
// made for one pass.
bool plan_general(const Problem &p, int cus, PlanChoice *pc, int *k_pass) {
  long long k_eff = std::max(p.K, 1);
  for (int iter = 0; iter < 8; ++iter) {
    *pc = plan(p.M, p.N, static_cast<int>(k_eff), cus, &p);
    const KernelInfo *k = find_kernel(pc->kernel);
    if (!dma_tile_usable(p, k->bm, k->bn, k->bk)) return false;
    auto fits = [&](long long kc) {
      const long long span = ceil_div(kc, k->bk) * k->bk + k->bk;
      return operand_fits(!p.ta, k->bm, p.lda, span) && operand_fits(p.tb, k->bn, p.ldb, span);
    };
    long long kp = k_eff;
    while (!fits(kp) && kp > k->bk) kp = std::max<long long>(k->bk, kp / 2 / k->bk * k->bk);
    if (!fits(kp)) return false;
    if (kp >= k_eff) {
      *k_pass = static_cast<int>(k_eff);
      return true;
    }
    k_eff = kp;
  }
  return false;
}

// Workspace of the general form: the largest of its passes' (the last pass
// may be shorter and split differently).
size_t general_workspace(const Problem &p, const PlanChoice &pc, int k_pass, int cus) {
  size_t need = 0;
  const int lens[2] = {std::min(k_pass, p.K), p.K > k_pass ? p.K % k_pass : 0};
  for (int len : lens) {
    Resolved r;
    if (len > 0 && resolve(p.M, p.N, len, pc.kernel, pc.split, pc.tail, cus, &r))
      need = std::max(need, workspace_for(p.M, p.N, r));
  }
  return need;
}

int run_general(Problem p, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = validate_general(p);
  if (st != GEMM_OK) return st;
  if (p.M == 0 || p.N == 0) return GEMM_OK;
  PlanChoice pc{0, 1, false};
  int k_pass = std::max(p.K, 1);
  const bool uses_ab = p.K > 0 && p.alpha != 0.0f;
  const int cus = planning_cus();
  if (uses_ab && !plan_general(p, cus, &pc, &k_pass)) return GEMM_ERR_INVALID_DIM;
  const size_t need = uses_ab ? general_workspace(p, pc, k_pass, cus) : 0;
  const bool own_ws = workspace == nullptr;
  if (!own_ws && workspace_bytes < need) return GEMM_ERR_WORKSPACE;

  int dev = 0, dev_cus = 0;
  st = check_device(&dev, &dev_cus);
  if (st != GEMM_OK) return st;
  if (!uses_ab) return launch_scale_c(p, cus, stream);
  // K passes: op(A)[:, k0:k0+kp] op(B)[k0:k0+kp, :], accumulated into C.
  auto passes = [&](void *ws) {
    const int split = ws || need == 0 ? pc.split : 1;   // no workspace to be had: no split
    const float beta0 = p.beta;
    for (int k0 = 0; k0 < p.K; k0 += k_pass) {
      Problem q = p;
      q.K = std::min(k_pass, p.K - k0);
      q.A = p.A + (p.ta ? (long long)k0 * p.lda : k0);
      q.B = p.B + (p.tb ? k0 : (long long)k0 * p.ldb);
      q.beta = k0 == 0 ? beta0 : 1.0f;
      Resolved r;
      if (!resolve(q.M, q.N, q.K, pc.kernel, split, pc.tail, cus, &r)) return (int)GEMM_ERR_INVALID_PLAN;
      const int s2 = launch(q, r, ws, cus, stream);
      if (s2 != GEMM_OK) return s2;
    }
    return (int)GEMM_OK;
  };
  if (own_ws && need > 0) return with_library_workspace(dev, need, stream, passes);
  return passes(workspace);
}

}  // namespace

extern "C" {

int gemm_f32(const float *A, const float *B, float *C, int M, int N, int K, hipStream_t stream) {
  return run(A, B, C, M, N, K, nullptr, nullptr, 0, Ws::kLibrary, stream);
}

size_t gemm_f32_workspace_bytes(int M, int N, int K) {
  if (M < 0 || N < 0 || K < 0) return 0;
  const int cus = planning_cus();
  const PlanChoice pc = plan(M, N, K, cus);
  Resolved r;
  if (!resolve(M, N, K, pc.kernel, pc.split, pc.tail, cus, &r)) return 0;
  return workspace_for(M, N, r);
}

int gemm_f32_noalloc(const float *A, const float *B, float *C, int M, int N, int K,
                     hipStream_t stream) {
  return run(A, B, C, M, N, K, nullptr, nullptr, 0, Ws::kScratch, stream);
}

size_t gemm_f32_noalloc_scratch_bytes(void) { return kScratchBytes; }

int gemm_f32_ex(const float *A, const float *B, float *C, int M, int N, int K, void *workspace,
                size_t workspace_bytes, hipStream_t stream) {
  return run(A, B, C, M, N, K, nullptr, workspace, workspace_bytes, Ws::kCaller, stream);
}

int gemm_f32_plan_cus(int M, int N, int K, int num_cus, gemm_plan_t *out) {
  if (!out) return GEMM_ERR_NULL_PTR;
  if (M < 0 || N < 0 || K < 0 || num_cus < 1) return GEMM_ERR_INVALID_DIM;
  const PlanChoice pc = plan(M, N, K, num_cus);
  Resolved r;
  if (!resolve(M, N, K, pc.kernel, pc.split, pc.tail, num_cus, &r)) return GEMM_ERR_INVALID_PLAN;
  out->kernel = pc.kernel;
  out->split_k = r.splits;
  out->k_chunk = r.k_chunk;
  out->split_tail = r.dp_tiles > 0 ? 1 : 0;
  return GEMM_OK;
}

int gemm_f32_plan(int M, int N, int K, gemm_plan_t *out) {
  if (!out) return GEMM_ERR_NULL_PTR;
  if (M < 0 || N < 0 || K < 0) return GEMM_ERR_INVALID_DIM;
  return gemm_f32_plan_cus(M, N, K, planning_cus(), out);
}

size_t gemm_f32_plan_workspace_bytes(int M, int N, int K, const gemm_plan_t *p) {
  if (!p || M < 0 || N < 0 || K < 0) return 0;
  PlanChoice pc{p->kernel, p->split_k, p->split_tail != 0};
  const int cus = planning_cus();
  if (pc.kernel == GEMM_KERNEL_AUTO) pc = plan(M, N, K, cus);
  else if (p->split_tail < 0 || p->split_tail > 1) return 0;
  Resolved r;
  if (!resolve(M, N, K, pc.kernel, pc.split, pc.tail, cus, &r)) return 0;
  return workspace_for(M, N, r);
}

int gemm_f32_with_plan(const float *A, const float *B, float *C, int M, int N, int K,
                       const gemm_plan_t *p, void *workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  if (!p) return GEMM_ERR_INVALID_PLAN;
  return run(A, B, C, M, N, K, p, workspace, workspace_bytes, Ws::kCaller, stream);
}

int gemm_f32_general(int trans_a, int trans_b, int M, int N, int K, float alpha, const float *A,
                     int lda, const float *B, int ldb, float beta, float *C, int ldc,
                     void *workspace, size_t workspace_bytes, hipStream_t stream) {
  const Problem p{trans_a != 0, trans_b != 0, M, N, K, alpha, beta, A, B, C, lda, ldb, ldc};
  return run_general(p, workspace, workspace_bytes, stream);
}

size_t gemm_f32_general_workspace_bytes(int trans_a, int trans_b, int M, int N, int K, int lda,
                                        int ldb) {
  // alpha = 1 and C pointer, ldc = N stand-ins: only the plan matters here.
  const Problem p{trans_a != 0, trans_b != 0, M, N, K, 1.0f, 0.0f, nullptr, nullptr, nullptr,
                  lda, ldb, std::max(N, 1)};
  if (M < 0 || N < 0 || K < 0) return 0;
  const int a_cols = p.ta ? M : K, b_cols = p.tb ? K : N;
  if (lda < std::max(1, a_cols) || ldb < std::max(1, b_cols)) return 0;
  if (M == 0 || N == 0 || K == 0) return 0;
  PlanChoice pc{0, 1, false};
  int k_pass = K;
  const int cus = planning_cus();
  if (!plan_general(p, cus, &pc, &k_pass)) return 0;
  return general_workspace(p, pc, k_pass, cus);
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
    case GEMM_ERR_CAPTURING:
      return "stream is capturing a graph and the plan needs the library's workspace "
             "(pass a workspace instead)";
    case GEMM_ERR_SCRATCH_LIMIT:
      return "the plan's split-K partial sums exceed the static scratch buffer of "
             "gemm_f32_noalloc (gemm_f32_noalloc_scratch_bytes)";
    default: return "unknown status";
  }
}

int gemm_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"

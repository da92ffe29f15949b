// Device code of libgemm: FP32 C = A x B for gfx950 (CDNA4, wave64).
//
// The blocked algorithm is the one the pages teach (hpc.payai.win lesson 10,
// section 2; yekq.top LeetGPU walkthrough, sections v2 and v4): each
// workgroup owns one output tile, walks K in steps of BK, stages an A slice
// and a B slice in on-chip memory with zero fill past the matrix edges, keeps
// the partial sums in registers and stores only the in-range outputs. What is
// gfx950-specific here:
//   - the per-lane register tile of the pages becomes the accumulator of
//     v_mfma_f32_32x32x2_f32 (a 32x32 FP32 block per wave per instruction);
//   - LDS is double buffered, so one barrier per K step guards both the
//     read-after-write and the write-after-read hazard the lesson's two
//     barriers guard (section 3): at step t waves read buffer t%2 and fill
//     buffer (t+1)%2, and the barrier at the end of step t orders both;
//   - every lane stays alive to every barrier; out-of-range elements are
//     loaded as 0.0f and out-of-range outputs are skipped at the store;
//   - workgroup -> tile mapping is aware of the 8 XCDs (see map_tile);
//   - split-K: a third index cuts K into contiguous ranges whose partial tiles
//     go to a workspace and are summed by splitk_reduce in fixed order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemm {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;  // 4 waves of 64 lanes per workgroup
constexpr int kXcds = 8;       // MI355X: 8 accelerator dies of 32 CUs each

struct TileCoord {
  int tm, tn, split;
};

// Workgroup id -> (tile row, tile column, K range).
//
// The dispatcher hands consecutive workgroup ids to the 8 XCDs round robin,
// and each XCD has its own L2. The first step renumbers ids so that each XCD
// receives one contiguous range of logical ids (a bijection for any count).
// Logical ids then run over K ranges slowest, and within one K range over
// tiles in groups of `group_m` tile rows, column by column inside a group, so
// that the workgroups resident on one XCD at one time share A row panels and
// B column panels in that XCD's L2.
__device__ inline TileCoord map_tile(int bid, int tiles_m, int tiles_n, int splits,
                                     int group_m) {
  const int total = tiles_m * tiles_n * splits;
  const int q = total / kXcds, r = total % kXcds;
  const int xcd = bid % kXcds, local = bid / kXcds;
  const int id = xcd * q + (xcd < r ? xcd : r) + local;
  const int tiles = tiles_m * tiles_n;
  TileCoord c;
  c.split = id / tiles;
  const int t = id - c.split * tiles;
  const int per_group = group_m * tiles_n;
  const int g = t / per_group;
  const int first_m = g * group_m;
  const int rows_left = tiles_m - first_m;
  const int gsize = rows_left < group_m ? rows_left : group_m;
  const int within = t - g * per_group;
  c.tm = first_m + within % gsize;
  c.tn = within / gsize;
  return c;
}

// ---------------------------------------------------------------------------
// FP32 MFMA kernel.
//
// BM x BN output tile per workgroup of 4 waves arranged WAVES_M x WAVES_N;
// each wave owns a WM x WN sub-tile made of (WM/32) x (WN/32) accumulator
// blocks of v_mfma_f32_32x32x2_f32.
//
// Operand layout of that instruction (CDNA3/CDNA4 ISA, matrix instructions):
// lane l supplies A[i = l % 32][kk = l / 32] and B[kk = l / 32][j = l % 32]
// for a 32x2 by 2x32 product; its 16 accumulator values are the outputs at
// column j = l % 32 and rows 8*(v/4) + 4*(l/32) + v%4, v = 0..15.
//
// Which real k index an instruction's kk slot carries is free, as long as A
// and B agree: within a K step of BK, instruction s (s = 0..BK/2-1) takes
// k = s for lanes 0-31 and k = BK/2 + s for lanes 32-63. A lane therefore
// reads BK/2 consecutive k of one A row (two 16-byte LDS reads) and one B
// column at BK/2 consecutive k.
//
// LDS layout per buffer: A row-major [BM][BK + 4] (the 4-float pad makes the
// 16-byte row reads of 16 consecutive rows cover all 64 banks once), B
// row-major [BK][BN + 4] (the pad puts the two half-waves, which read rows
// BK/2 apart, on disjoint bank halves).
//
// VA / VB: 4 = 16-byte global loads (needs K % 4 == 0, resp. N % 4 == 0 and
// 16-byte aligned base pointers), 1 = 4-byte loads for any shape.
// CHECK = false only when the tile grid covers M and N exactly and every K
// range is a whole number of K steps; otherwise each load is predicated and
// zero-filled and each store is predicated.
template <int BM, int BN, int BK, int WAVES_M, int WAVES_N>
struct MfmaShape {
  static constexpr int WM = BM / WAVES_M;
  static constexpr int WN = BN / WAVES_N;
  static constexpr int FM = WM / 32;
  static constexpr int FN = WN / 32;
  static constexpr int KH = BK / 2;
  static constexpr int LDA = BK + 4;
  static constexpr int LDB = BN + 4;
  static_assert(WAVES_M * WAVES_N == 4, "4 waves per workgroup");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile is whole 32x32 blocks");
  static_assert(BK % 8 == 0, "BK/2 k-steps, read in 16-byte groups");
};

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int VA, int VB, bool CHECK,
          int MIN_WAVES>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(MIN_WAVES, MIN_WAVES == 1 ? 1 : 8)))
void mfma_gemm_kernel(const float *__restrict__ A, const float *__restrict__ B,
                      float *__restrict__ C, int M, int N, int K, int k_chunk,
                      int tiles_m, int tiles_n, int splits, long long slab) {
  using S = MfmaShape<BM, BN, BK, WAVES_M, WAVES_N>;
  constexpr int FM = S::FM, FN = S::FN, KH = S::KH, LDA = S::LDA, LDB = S::LDB;
  constexpr int A_CPR = BK / VA;              // load chunks per A tile row
  constexpr int A_PER_T = BM * A_CPR / kThreads;
  constexpr int B_CPR = BN / VB;              // load chunks per B tile row
  constexpr int B_PER_T = BK * B_CPR / kThreads;
  static_assert(BM * A_CPR % kThreads == 0 && BK * B_CPR % kThreads == 0, "even load split");

  __shared__ __attribute__((aligned(16))) float As[2][BM * LDA];
  __shared__ __attribute__((aligned(16))) float Bs[2][BK * LDB];

  const TileCoord tc = map_tile(blockIdx.x, tiles_m, tiles_n, splits, 8);
  const int m0 = tc.tm * BM, n0 = tc.tn * BN;
  const int k_begin = tc.split * k_chunk;
  const int k_end = min(K, k_begin + k_chunk);
  const int nk = (k_end - k_begin + BK - 1) / BK;
  float *__restrict__ Cout = C + (long long)tc.split * slab;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int half = lane >> 5;   // which k half of the K step this lane carries
  const int l32 = lane & 31;

  // Per-thread global source pointers at the first K step, and LDS offsets.
  const float *pa[A_PER_T];
  int a_lds[A_PER_T];
  bool a_row_ok[A_PER_T];
  int a_k[A_PER_T];
#pragma unroll
  for (int i = 0; i < A_PER_T; ++i) {
    const int e = tid + kThreads * i;
    const int r = e / A_CPR, c = e % A_CPR;
    const int row = m0 + r;
    a_row_ok[i] = !CHECK || row < M;
    const int row_c = (CHECK && row >= M) ? (M - 1) : row;
    a_k[i] = k_begin + c * VA;
    pa[i] = A + (long long)row_c * K + a_k[i];
    a_lds[i] = r * LDA + c * VA;
  }
  const float *pb[B_PER_T];
  int b_lds[B_PER_T];
  bool b_col_ok[B_PER_T];
  int b_k[B_PER_T];
#pragma unroll
  for (int i = 0; i < B_PER_T; ++i) {
    const int e = tid + kThreads * i;
    const int r = e / B_CPR, c = e % B_CPR;
    const int col = n0 + c * VB;
    b_col_ok[i] = !CHECK || col < N;
    const int col_c = (CHECK && col >= N) ? 0 : col;
    b_k[i] = k_begin + r;
    const int row_c = (CHECK && b_k[i] >= K) ? 0 : b_k[i];
    pb[i] = B + (long long)row_c * N + col_c;
    b_lds[i] = r * LDB + c * VB;
  }

  floatx4 ra[A_PER_T * VA / 4 + (VA == 1 ? 1 : 0)];
  float ra1[VA == 1 ? A_PER_T : 1];
  floatx4 rb[B_PER_T * VB / 4 + (VB == 1 ? 1 : 0)];
  float rb1[VB == 1 ? B_PER_T : 1];
  (void)ra; (void)ra1; (void)rb; (void)rb1;

  // Global -> registers for K step starting at k_off (relative to k_begin).
  auto load_global = [&](int k_off) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const bool ok = a_row_ok[i] && (!CHECK || a_k[i] + k_off < k_end);
      if constexpr (VA == 4) {
        ra[i] = ok ? *reinterpret_cast<const floatx4 *>(pa[i] + k_off) : floatx4{0.f, 0.f, 0.f, 0.f};
      } else {
        ra1[i] = ok ? pa[i][k_off] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const bool ok = b_col_ok[i] && (!CHECK || b_k[i] + k_off < k_end);
      const long long off = (long long)k_off * N;
      if constexpr (VB == 4) {
        rb[i] = ok ? *reinterpret_cast<const floatx4 *>(pb[i] + off) : floatx4{0.f, 0.f, 0.f, 0.f};
      } else {
        rb1[i] = ok ? pb[i][off] : 0.f;
      }
    }
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      if constexpr (VA == 4) {
        *reinterpret_cast<floatx4 *>(&As[buf][a_lds[i]]) = ra[i];
      } else {
        As[buf][a_lds[i]] = ra1[i];
      }
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      if constexpr (VB == 4) {
        *reinterpret_cast<floatx4 *>(&Bs[buf][b_lds[i]]) = rb[i];
      } else {
        Bs[buf][b_lds[i]] = rb1[i];
      }
    }
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  load_global(0);
  store_lds(0);
  __syncthreads();

  for (int t = 0; t < nk; ++t) {
    const int cur = t & 1;
    const bool more = t + 1 < nk;
    if (more) load_global((t + 1) * BK);

    float a[FM][KH];
    float b[FN][KH];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const float *src = &As[cur][(wm * S::WM + fm * 32 + l32) * LDA + half * KH];
#pragma unroll
      for (int s = 0; s < KH; s += 4) {
        const floatx4 v = *reinterpret_cast<const floatx4 *>(src + s);
        a[fm][s] = v[0]; a[fm][s + 1] = v[1]; a[fm][s + 2] = v[2]; a[fm][s + 3] = v[3];
      }
    }
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const float *src = &Bs[cur][(half * KH) * LDB + wn * S::WN + fn * 32 + l32];
#pragma unroll
      for (int s = 0; s < KH; ++s) b[fn][s] = src[s * LDB];
    }
#pragma unroll
    for (int s = 0; s < KH; ++s)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[fm][s], b[fn][s], acc[fm][fn], 0, 0, 0);

    if (more) store_lds(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds column l32 of each 32x32 block, rows 8*(v/4) + 4*half + v%4.
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int col = n0 + wn * S::WN + fn * 32 + l32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * S::WM + fm * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        if (!CHECK || (row < M && col < N)) Cout[(long long)row * N + col] = acc[fm][fn][v];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Vector-FMA kernel: 64x64 tile, K step 16, each of the 256 lanes owns a 4x4
// register tile (the two-dimensional register coarsening of the yekq.top
// walkthrough, section v4, laid out for wave64). A is stored transposed in
// LDS ([k][m]) so a lane reads its 4 rows of A as one 16-byte read, B
// row-major ([k][n]) so it reads its 4 columns likewise. Single LDS buffer
// with the lesson's two barriers per K step.
template <bool CHECK>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads)))
void valu_gemm_kernel(const float *__restrict__ A, const float *__restrict__ B,
                      float *__restrict__ C, int M, int N, int K, int k_chunk, int tiles_m,
                      int tiles_n, int splits, long long slab) {
  constexpr int BM = 64, BN = 64, BK = 16, LD = 64 + 4;
  __shared__ __attribute__((aligned(16))) float At[BK * LD];
  __shared__ __attribute__((aligned(16))) float Bs[BK * LD];

  const TileCoord tc = map_tile(blockIdx.x, tiles_m, tiles_n, splits, 8);
  const int m0 = tc.tm * BM, n0 = tc.tn * BN;
  const int k_begin = tc.split * k_chunk;
  const int k_end = min(K, k_begin + k_chunk);
  float *__restrict__ Cout = C + (long long)tc.split * slab;

  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;  // lane tile at rows 4*ty.., cols 4*tx..

  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  for (int k0 = k_begin; k0 < k_end; k0 += BK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + kThreads * i;
      const int r = e >> 4, kk = e & 15;     // A: 64 rows x 16 k, lanes along k
      const int row = m0 + r, k = k0 + kk;
      At[kk * LD + r] = (!CHECK || (row < M && k < k_end)) ? A[(long long)row * K + k] : 0.0f;
      const int kr = e >> 6, cc = e & 63;    // B: 16 k x 64 cols, lanes along n
      const int kb = k0 + kr, col = n0 + cc;
      Bs[kr * LD + cc] = (!CHECK || (kb < k_end && col < N)) ? B[(long long)kb * N + col] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      const floatx4 av = *reinterpret_cast<const floatx4 *>(&At[kk * LD + 4 * ty]);
      const floatx4 bv = *reinterpret_cast<const floatx4 *>(&Bs[kk * LD + 4 * tx]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + 4 * ty + i;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + 4 * tx + j;
      if (!CHECK || (row < M && col < N)) Cout[(long long)row * N + col] = acc[i][j];
    }
  }
}

// ---------------------------------------------------------------------------
// Split-K reduction: C[e] = ws[0][e] + ws[1][e] + ... + ws[S-1][e], always in
// ascending slab order, so the result does not depend on which workgroup
// finished first. Pure streaming: S*M*N reads and M*N writes, HBM bound.
template <int V>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads)))
void splitk_reduce_kernel(const float *__restrict__ ws, float *__restrict__ C, long long count,
                          int splits) {
  const long long stride = (long long)gridDim.x * kThreads;
  for (long long e = (long long)blockIdx.x * kThreads + threadIdx.x; e * V < count; e += stride) {
    if constexpr (V == 4) {
      floatx4 s = *reinterpret_cast<const floatx4 *>(ws + e * 4);
      for (int p = 1; p < splits; ++p) {
        const floatx4 v = *reinterpret_cast<const floatx4 *>(ws + (long long)p * count + e * 4);
        s[0] = s[0] + v[0]; s[1] = s[1] + v[1]; s[2] = s[2] + v[2]; s[3] = s[3] + v[3];
      }
      *reinterpret_cast<floatx4 *>(C + e * 4) = s;
    } else {
      float s = ws[e];
      for (int p = 1; p < splits; ++p) s = s + ws[(long long)p * count + e];
      C[e] = s;
    }
  }
}

// Fill C with +0.0 (the K = 0 product).
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads)))
void fill_zero_kernel(float *__restrict__ C, long long count) {
  const long long stride = (long long)gridDim.x * kThreads;
  for (long long e = (long long)blockIdx.x * kThreads + threadIdx.x; e < count; e += stride)
    C[e] = 0.0f;
}

}  // namespace gemm

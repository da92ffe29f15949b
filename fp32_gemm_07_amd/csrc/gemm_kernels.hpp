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
//   - one barrier per K step guards both the read-after-write and the
//     write-after-read hazard the lesson's two barriers guard (section 3):
//     the register-staged kernel double-buffers LDS (at step t waves read
//     buffer t%2 and fill buffer (t+1)%2), the copy-fed kernel rotates a ring
//     of 3 or 4 stages filled by direct global -> LDS copies;
//   - every lane stays alive to every barrier; out-of-range elements are
//     loaded as 0.0f and out-of-range outputs are skipped at the store;
//   - workgroup -> tile mapping is aware of the 8 XCDs (see map_tile);
//   - split-K: a third index cuts K into contiguous ranges whose partial tiles
//     go to a workspace and are summed in fixed order (splitk_reduce_kernel);
//     the copy-fed kernel can also split only the tiles of the last, partial
//     round of workgroups and compute the others whole (tail_reduce_kernel).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gemm {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;  // 4 waves of 64 lanes per workgroup
constexpr int kXcds = 8;       // MI355X: 8 accelerator dies of 32 CUs each

constexpr int kGroupM = 8;     // tile rows per group of the tile order

struct TileCoord {
  int tm, tn, split;
  int whole;   // 1: the tile's whole K range, stored into C
};

// The dispatcher hands consecutive workgroup ids to the 8 XCDs round robin,
// and each XCD has its own L2. This renumbering of ids 0 .. total-1 gives
// each XCD one contiguous range of logical ids (a bijection for any count).
__device__ inline int xcd_order(int bid, int total) {
  const unsigned ut = static_cast<unsigned>(total), ub = static_cast<unsigned>(bid);
  const int q = static_cast<int>(ut / kXcds), r = static_cast<int>(ut % kXcds);
  const int xcd = static_cast<int>(ub % kXcds), local = static_cast<int>(ub / kXcds);
  return xcd * q + (xcd < r ? xcd : r) + local;
}

// Tile order: tiles in groups of `group_m` tile rows, column by column inside
// a group, so that the workgroups resident on one XCD at one time share A row
// panels and B column panels in that XCD's L2. Tile t -> (tile row, column).
__device__ inline void grouped_tile(int t, int tiles_m, int tiles_n, int group_m, int *tm,
                                    int *tn) {
  const int per_group = group_m * tiles_n;
  const int g = t / per_group;
  const int first_m = g * group_m;
  const int rows_left = tiles_m - first_m;
  const int gsize = rows_left < group_m ? rows_left : group_m;
  const int within = t - g * per_group;
  *tm = first_m + within % gsize;
  *tn = within / gsize;
}

// Division by a divisor fixed for a launch, without the ~30-instruction
// integer division sequence: for 1 <= d < 2^31, with s = ceil(log2 d) and
// m = ceil(2^(31+s) / d) (below 2^32), floor(n / d) = (n * m) >> (31 + s) for
// every 0 <= n < 2^31. Writing m*d = 2^(31+s) + e with 0 <= e < d,
// n * m / 2^(31+s) = n / d + n*e / (d * 2^(31+s)), and the second term is
// below 2^-s <= 1/d, too little to reach the next integer. The host computes
// m and s once per launch (make_fast_div).
struct FastDiv {
  unsigned mul;
  unsigned shift;   // 31 + s
};

inline FastDiv make_fast_div(int d) {
  unsigned s = 0;
  while ((1LL << s) < d) ++s;
  const unsigned long long p = 1ULL << (31 + s);
  return FastDiv{static_cast<unsigned>((p + static_cast<unsigned>(d) - 1) / static_cast<unsigned>(d)),
                 31 + s};
}

__device__ inline int fast_div(int n, const FastDiv &d) {
  return static_cast<int>((static_cast<unsigned long long>(static_cast<unsigned>(n)) * d.mul) >>
                          d.shift);
}

// The tile order of one launch, with the divisors of its grouped order
// prepared on the host (map_tile_fast, grouped_tile_fast: the same mapping as
// map_tile and grouped_tile below, which divide at run time).
struct TileOrder {
  int tiles_m, tiles_n, splits, dp_tiles;
  FastDiv per_group;   // kGroupM * tiles_n tiles per group of tile rows
  FastDiv last_rows;   // tile rows of the last group (kGroupM when it is whole)
};

inline TileOrder make_tile_order(int tiles_m, int tiles_n, int splits, int dp_tiles) {
  const int last = tiles_m % kGroupM;
  return TileOrder{tiles_m, tiles_n, splits, dp_tiles, make_fast_div(kGroupM * tiles_n),
                   make_fast_div(last ? last : kGroupM)};
}

// The copy-fed kernel's scalar form of a tile order. Without a split every
// tile is whole, and the whole-tile path of map_tile_fast maps workgroup ids
// exactly as the split path does with one K range (xcd_order over all tiles),
// so dp_tiles becomes the tile count and that path needs neither the split
// count nor its divisor.
struct KernelOrder {
  int dp_tiles;
  unsigned group_mul, rows_mul, shifts;
  int splits;
};

inline KernelOrder kernel_order(const TileOrder &o) {
  return KernelOrder{o.splits == 1 ? o.tiles_m * o.tiles_n : o.dp_tiles, o.per_group.mul,
                     o.last_rows.mul, o.per_group.shift | (o.last_rows.shift << 8), o.splits};
}

__device__ inline void grouped_tile_fast(int t, const TileOrder &o, int *tm, int *tn) {
  const int g = fast_div(t, o.per_group);
  const int first_m = g * kGroupM;
  const int within = t - g * (kGroupM * o.tiles_n);
  if (o.tiles_m - first_m >= kGroupM) {
    *tm = first_m + within % kGroupM;
    *tn = within / kGroupM;
  } else {
    const int q = fast_div(within, o.last_rows);
    *tm = first_m + (within - q * (o.tiles_m - first_m));
    *tn = q;
  }
}

// Workgroup id -> (tile row, tile column, K range).
//
// The first `dp_tiles` tiles of the tile order are computed whole, one
// workgroup each (ids 0 .. dp_tiles-1); every later tile is cut into `splits`
// K ranges, one workgroup each (the ids after). With dp_tiles = 0 every tile
// is split (plain split-K; splits = 1: one workgroup per tile). Within each
// of the two id ranges ids are renumbered per XCD (xcd_order), and the split
// part runs over K ranges slowest.
__device__ inline TileCoord map_tile(int bid, int tiles_m, int tiles_n, int splits, int group_m,
                                     int dp_tiles = 0) {
  TileCoord c;
  int t;
  if (bid < dp_tiles) {
    t = xcd_order(bid, dp_tiles);
    c.split = 0;
    c.whole = 1;
  } else {
    const int tail = tiles_m * tiles_n - dp_tiles;
    const int id = xcd_order(bid - dp_tiles, tail * splits);
    c.split = id / tail;
    t = dp_tiles + (id - c.split * tail);
    c.whole = splits == 1;
  }
  grouped_tile(t, tiles_m, tiles_n, group_m, &c.tm, &c.tn);
  return c;
}

// map_tile with group_m = kGroupM and the divisors of a TileOrder.
__device__ inline TileCoord map_tile_fast(int bid, const TileOrder &o) {
  TileCoord c;
  int t;
  if (bid < o.dp_tiles) {
    t = xcd_order(bid, o.dp_tiles);
    c.split = 0;
    c.whole = 1;
  } else {
    // Split tiles (large products only, where a run-time division costs
    // nothing that shows).
    const int tail = o.tiles_m * o.tiles_n - o.dp_tiles;
    const int id = xcd_order(bid - o.dp_tiles, tail * o.splits);
    c.split = o.splits == 1 ? 0 : id / tail;
    t = o.dp_tiles + (id - c.split * tail);
    c.whole = o.splits == 1;
  }
  grouped_tile_fast(t, o, &c.tm, &c.tn);
  return c;
}

// ---------------------------------------------------------------------------
// FP32 MFMA kernel.
//
// BM x BN output tile per workgroup of 1, 2, 4 or 8 waves arranged WAVES_M x
// WAVES_N; each wave owns a WM x WN sub-tile made of (WM/MI) x (WN/MI)
// accumulator blocks of one FP32 matrix instruction. With one wave per
// workgroup the wave stages its own tiles and never waits on another wave
// (the barrier of a one-wave workgroup is free), and several such workgroups
// share a CU, one per SIMD.
//   MI = 32: v_mfma_f32_32x32x2_f32 (32x2 by 2x32, 16 accumulators per lane);
//   MI = 16: v_mfma_f32_16x16x4_f32 (16x4 by 4x16, 4 accumulators per lane).
// Both retire 256 FLOP per clock per CU.
//
// Operand layout (CDNA3/CDNA4 ISA, matrix instructions): the 64 lanes form
// NQ = 64/MI groups q = lane / MI of MI lanes each; lane (q, i) supplies
// A[row i][kk = q] and B[kk = q][column i]. Accumulator v of lane (q, i)
// holds output column i and row 8*(v/4) + 4*q + v%4 (MI = 32) or
// 4*q + v (MI = 16).
//
// Which real k index a group's kk slot carries is free, as long as A and B
// agree: within a K step of BK, instruction s (s = 0..KS-1, KS = BK/NQ) takes
// k = q*KS + s for lane group q. A lane therefore reads KS consecutive k of
// one A row (one 16-byte LDS read per 4 instructions) and one B column at KS
// consecutive k.
//
// LDS layout per buffer: A row-major [BM][BK + 4], B row-major [BK][BN + 4];
// the pads shift consecutive rows across banks.
//
// VA / VB: 4 = 16-byte global loads (needs K % 4 == 0, resp. N % 4 == 0 and
// 16-byte aligned base pointers), 1 = 4-byte loads for any shape.
// CHECK = false only when the tile grid covers M and N exactly and every K
// range is a whole number of K steps; otherwise each load is predicated and
// zero-filled and each store is predicated.
template <int MI, int BM, int BN, int BK, int WAVES_M, int WAVES_N>
struct MfmaShape {
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = 64 * NWAVES;
  static constexpr int NQ = 64 / MI;    // lane groups = k per instruction
  static constexpr int ACC = MI * MI / 64;  // accumulators per lane per block
  static constexpr int WM = BM / WAVES_M;
  static constexpr int WN = BN / WAVES_N;
  static constexpr int FM = WM / MI;
  static constexpr int FN = WN / MI;
  static constexpr int KS = BK / NQ;    // instructions per K step
  static constexpr int NG = KS / 4;     // fragment groups of 4 instructions per K step
  static constexpr int LDA = BK + 4;
  static constexpr int LDB = BN + 4;
  static_assert(MI == 16 || MI == 32, "16x16x4 or 32x32x2 FP32 MFMA");
  static_assert(NWAVES == 1 || NWAVES == 2 || NWAVES == 4 || NWAVES == 8,
                "1, 2, 4 or 8 waves per workgroup");
  static_assert(WM % MI == 0 && WN % MI == 0, "wave tile is whole blocks");
  static_assert(KS % 4 == 0 && (NG == 1 || NG % 2 == 0),
                "K step is one or an even number of 4-instruction groups");
};

template <int MI>
struct Mfma;
template <>
struct Mfma<32> {
  typedef floatx16 acc_t;
  static __device__ inline acc_t run(float a, float b, const acc_t &c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  // output row of accumulator v for lane group q
  static __device__ inline int row(int q, int v) { return 8 * (v >> 2) + 4 * q + (v & 3); }
};
template <>
struct Mfma<16> {
  typedef floatx4 acc_t;
  static __device__ inline acc_t run(float a, float b, const acc_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ inline int row(int q, int v) { return 4 * q + v; }
};

// Software pipeline of one K step t (buffer cur = t % 2), NG groups g of 4
// instructions, fragments double buffered in registers (slot = g % 2):
//   group g < NG-1: MFMAs of instruction 4g, then LDS reads of group g+1's
//                   fragments, then the MFMAs of instructions 4g+1..4g+3;
//   group NG-1:     (all reads of buffer cur are issued) store the staged
//                   global data of step t+1 into buffer cur^1, barrier, MFMAs
//                   of instruction 4g, then read group 0 of step t+1 from
//                   buffer cur^1 and issue the global loads of step t+2, then
//                   the remaining MFMAs.
// Each fragment read has at least 3 x FM x FN MFMAs to land, each global load
// a whole K step, and the barrier and LDS stores sit where the matrix pipe
// still has queued work. __builtin_amdgcn_sched_barrier(0) keeps the compiler
// from regrouping the segments.
template <int MI, int BM, int BN, int BK, int WAVES_M, int WAVES_N, int VA, int VB, bool CHECK,
          int WAVES_PER_EU>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WAVES_M * WAVES_N,
                                                      64 * WAVES_M * WAVES_N),
                          amdgpu_waves_per_eu(WAVES_PER_EU, WAVES_PER_EU)))
void mfma_gemm_kernel(const float *__restrict__ A, const float *__restrict__ B,
                      float *__restrict__ C, int M, int N, int K, int k_chunk,
                      int tiles_m, int tiles_n, int splits, long long slab) {
  using S = MfmaShape<MI, BM, BN, BK, WAVES_M, WAVES_N>;
  using Op = Mfma<MI>;
  using acc_t = typename Op::acc_t;
  constexpr int T = S::THREADS;
  constexpr int FM = S::FM, FN = S::FN, KS = S::KS, NG = S::NG, LDA = S::LDA, LDB = S::LDB;
  constexpr int A_CPR = BK / VA;              // load chunks per A tile row
  constexpr int A_PER_T = BM * A_CPR / T;
  constexpr int B_CPR = BN / VB;              // load chunks per B tile row
  constexpr int B_PER_T = BK * B_CPR / T;
  static_assert(BM * A_CPR % T == 0 && BK * B_CPR % T == 0, "even load split");

  __shared__ __attribute__((aligned(16))) float As[2][BM * LDA];
  __shared__ __attribute__((aligned(16))) float Bs[2][BK * LDB];

  const TileCoord tc = map_tile(blockIdx.x, tiles_m, tiles_n, splits, kGroupM);
  const int m0 = tc.tm * BM, n0 = tc.tn * BN;
  const int k_begin = tc.split * k_chunk;
  const int k_end = min(K, k_begin + k_chunk);
  const int nk = (k_end - k_begin + BK - 1) / BK;
  float *__restrict__ Cout = C + (long long)tc.split * slab;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int q = lane / MI;       // lane group: which k slot of each instruction
  const int li = lane % MI;      // row of A / column of B within a block

  // Loads: the tile is CPR chunks (of VA or VB floats) per row; load i of
  // thread tid takes chunk e = tid + T*i in row-major chunk order. Either a
  // pass of the workgroup covers whole rows (T % CPR == 0: row r0 + i*T/CPR,
  // fixed chunk) or a row takes several passes (CPR % T == 0: row i/(CPR/T),
  // chunk tid + T*(i % (CPR/T))). Either way the per-load offsets from one
  // base pointer per operand are uniform across the workgroup.
  static_assert((T % A_CPR == 0 || A_CPR % T == 0) && (T % B_CPR == 0 || B_CPR % T == 0),
                "load chunks tile the rows evenly");
  constexpr bool A_WHOLE = T % A_CPR == 0, B_WHOLE = T % B_CPR == 0;
  constexpr int A_RPP = A_WHOLE ? T / A_CPR : 1;   // rows per pass
  constexpr int A_PPR = A_WHOLE ? 1 : A_CPR / T;   // passes per row
  constexpr int B_RPP = B_WHOLE ? T / B_CPR : 1;
  constexpr int B_PPR = B_WHOLE ? 1 : B_CPR / T;
  auto a_row = [](int i) { return A_WHOLE ? i * A_RPP : i / A_PPR; };
  auto a_col = [](int i) { return A_WHOLE ? 0 : T * (i % A_PPR) * VA; };
  auto b_row = [](int i) { return B_WHOLE ? i * B_RPP : i / B_PPR; };
  auto b_col = [](int i) { return B_WHOLE ? 0 : T * (i % B_PPR) * VB; };
  const int ar0 = A_WHOLE ? tid / A_CPR : 0, ac = (A_WHOLE ? tid % A_CPR : tid) * VA;
  const int br0 = B_WHOLE ? tid / B_CPR : 0, bc = (B_WHOLE ? tid % B_CPR : tid) * VB;
  const float *pa = A + (long long)(m0 + ar0) * K + (k_begin + ac);
  const float *pb = B + (long long)(k_begin + br0) * N + (n0 + bc);
  const int a_lds = ar0 * LDA + ac;
  const int b_lds = br0 * LDB + bc;

  floatx4 ra[VA == 4 ? A_PER_T : 1];
  float ra1[VA == 1 ? A_PER_T : 1];
  floatx4 rb[VB == 4 ? B_PER_T : 1];
  float rb1[VB == 1 ? B_PER_T : 1];
  (void)ra; (void)ra1; (void)rb; (void)rb1;

  // Global -> registers for the K step starting at k_off (relative to k_begin).
  auto load_global = [&](int k_off) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const bool ok = !CHECK || (k_begin + ac + a_col(i) + k_off < k_end && m0 + ar0 + a_row(i) < M);
      const float *p = pa + (long long)a_row(i) * K + a_col(i) + k_off;
      if constexpr (VA == 4) {
        ra[i] = ok ? *reinterpret_cast<const floatx4 *>(p) : floatx4{0.f, 0.f, 0.f, 0.f};
      } else {
        ra1[i] = ok ? *p : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const bool ok =
          !CHECK || (n0 + bc + b_col(i) < N && k_begin + br0 + b_row(i) + k_off < k_end);
      const float *p = pb + (long long)(b_row(i) + k_off) * N + b_col(i);
      if constexpr (VB == 4) {
        rb[i] = ok ? *reinterpret_cast<const floatx4 *>(p) : floatx4{0.f, 0.f, 0.f, 0.f};
      } else {
        rb1[i] = ok ? *p : 0.f;
      }
    }
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PER_T; ++i) {
      const int off = a_lds + a_row(i) * LDA + a_col(i);
      if constexpr (VA == 4) {
        *reinterpret_cast<floatx4 *>(&As[buf][off]) = ra[i];
      } else {
        As[buf][off] = ra1[i];
      }
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; ++i) {
      const int off = b_lds + b_row(i) * LDB + b_col(i);
      if constexpr (VB == 4) {
        *reinterpret_cast<floatx4 *>(&Bs[buf][off]) = rb[i];
      } else {
        Bs[buf][off] = rb1[i];
      }
    }
  };

  // Fragments of one group (4 instructions): per block row of A one 16-byte
  // read of 4 consecutive k; per block column of B 4 single reads.
  floatx4 fa[2][FM];
  float fb[2][FN][4];
  const int a_frag_off = (wm * S::WM + li) * LDA + q * KS;
  const int b_frag_off = (q * KS) * LDB + wn * S::WN + li;
  auto load_frags = [&](int buf, int g, int slot) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
      fa[slot][fm] = *reinterpret_cast<const floatx4 *>(&As[buf][a_frag_off + fm * MI * LDA + 4 * g]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        fb[slot][fn][j] = Bs[buf][b_frag_off + (4 * g + j) * LDB + fn * MI];
  };

  acc_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < S::ACC; ++v) acc[i][j][v] = 0.0f;

  auto mfma_step = [&](int slot, int j) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        acc[fm][fn] = Op::run(fa[slot][fm][j], fb[slot][fn][j], acc[fm][fn]);
  };

  // Prologue: K step 0 into buffer 0, its first fragments, K step 1 in flight.
  load_global(0);
  store_lds(0);
  __syncthreads();
  load_frags(0, 0, 0);
  if (nk > 1) load_global(BK);

  // One K step. The fragment slot of group g of step t is (t * NG + g) % 2;
  // it must be a compile-time constant (registers cannot be indexed), so when
  // NG is odd the step loop is unrolled by two and P = t % 2 is passed in.
  auto k_step = [&](int t, auto parity) {
    constexpr int P = decltype(parity)::value;
    const int cur = t & 1;
    const bool more = t + 1 < nk;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int slot = (P * NG + g) & 1;
      if (g < NG - 1) {
        mfma_step(slot, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_frags(cur, g + 1, slot ^ 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 1; j < 4; ++j) mfma_step(slot, j);
        __builtin_amdgcn_sched_barrier(0);
      } else {
        if (more) store_lds(cur ^ 1);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        mfma_step(slot, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (more) {
          load_frags(cur ^ 1, 0, slot ^ 1);
          if (t + 2 < nk) load_global((t + 2) * BK);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 1; j < 4; ++j) mfma_step(slot, j);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  if constexpr (NG % 2 == 0) {
    for (int t = 0; t < nk; ++t) k_step(t, std::integral_constant<int, 0>());
  } else {
    for (int t = 0; t < nk; t += 2) {
      k_step(t, std::integral_constant<int, 0>());
      if (t + 1 < nk) k_step(t + 1, std::integral_constant<int, 1>());
    }
  }

  // Epilogue: accumulator v of block (fm, fn) is output row Op::row(q, v) and
  // column li of that block.
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int col = n0 + wn * S::WN + fn * MI + li;
#pragma unroll
      for (int v = 0; v < S::ACC; ++v) {
        const int row = m0 + wm * S::WM + fm * MI + Op::row(q, v);
        if (!CHECK || (row < M && col < N)) Cout[(long long)row * N + col] = acc[fm][fn][v];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// FP32 MFMA kernel fed by direct global -> LDS copies.
//
// gfx950's buffer_load_dwordx4 ... lds copies 16 bytes per lane from global
// memory straight into LDS (lane i's bytes land at M0 + 16*i), so no operand
// data passes through registers: no staging VGPRs, no LDS store
// instructions, and a wave only waits for a K step's data when it is about
// to consume it. K steps rotate through NS LDS stages. Each copy goes through
// a buffer resource whose range check (per dword) turns an out-of-range
// offset into zeros; lanes whose chunk lies outside the matrix, or past the
// end of the K range, get such an offset, which is the zero fill of the
// edges. The 16-byte copies only need 4-byte aligned sources, so rows of any
// length and any row stride are copied this way; a chunk that straddles the
// end of the K range in a K-contiguous operand has its trailing floats zeroed
// in LDS (zero_k_tail), and chunks straddling the last row or column of the
// output only feed outputs that are never stored.
//
// Each operand is stored one of two ways (DmaOperand):
//   K-contiguous (A as given, or B given transposed): element (x, k) of the
//     operand at x*ld + k. LDS [BX][BK]; 16-byte chunk c of row x is stored
//     at chunk c ^ swz_k(x), so the 16-byte fragment reads of 16 consecutive
//     rows hit distinct banks; a lane's fragment is one 16-byte read of 4
//     consecutive k.
//   M/N-contiguous (B as given, or A given transposed): element (x, k) at
//     k*ld + x. LDS [BK][BX]; the chunks of row k are flipped by
//     ((k / KS) % NQ) * MI floats, so the NQ lane groups of an instruction,
//     which read rows KS apart, land MI floats apart, on different banks; a
//     lane's fragment is four 4-byte reads.
// Because a copy lands in LDS exactly as the 64 lanes are ordered, rows
// cannot be padded, hence the swizzles. The copies are issued with inline
// assembly: the compiler does not model the LDS write of its own builtin for
// this instruction, so the asm carries a memory clobber and the waits
// (s_waitcnt vmcnt) are explicit.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource: base address, byte range [0, bytes) (each dword of a
// load is checked on its own: dwords at or past the range read as zero), 32-bit
// data. bytes is capped at 2^31 so that kOutOfRange is always past the range.
__device__ inline u32x4 make_buffer_rsrc(const void *base, long long bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  u32x4 r;
  r[0] = static_cast<unsigned>(a);
  r[1] = static_cast<unsigned>(a >> 32) & 0xffffu;  // stride 0: raw byte buffer
  // The clamp in five scalar instructions on the two halves: written in C++,
  // the compiler turns it into 64-bit ordered compares, which run on the
  // vector unit and cost several times as many instructions.
  const unsigned lo = static_cast<unsigned>(bytes);
  const unsigned hi = static_cast<unsigned>(static_cast<unsigned long long>(bytes) >> 32);
  unsigned range;
  asm("s_cmp_lg_u32 %1, 0\n\t"
      "s_cselect_b32 %0, 0x80000000, %2\n\t"   // high half set: 2^31 or more (or negative)
      "s_min_u32 %0, %0, 0x80000000\n\t"
      "s_cmp_lt_i32 %1, 0\n\t"
      "s_cselect_b32 %0, 0, %0"                   // negative: empty
      : "=&s"(range)
      : "s"(hi), "s"(lo)
      : "scc");
  r[2] = range;
  r[3] = 0x00020000u;                               // 32-bit data, raw access
  return r;
}
constexpr unsigned kOutOfRange = 0x80000000u;

// The resource and the LDS address are the same for every lane. The
// compiler's divergence analysis does not always see that (values reached
// through captured references), and an "s" operand it believes divergent
// would be given vector registers; readfirstlane states the uniformity
// (and folds away where the compiler already knows it).
__device__ inline u32x4 uniform_rsrc(const u32x4 &r) {
  u32x4 u;
  u[0] = __builtin_amdgcn_readfirstlane(r[0]);
  u[1] = __builtin_amdgcn_readfirstlane(r[1]);
  u[2] = __builtin_amdgcn_readfirstlane(r[2]);
  u[3] = __builtin_amdgcn_readfirstlane(r[3]);
  return u;
}

// One copy instruction: each lane moves VEC floats (16 or 4 bytes) from
// rsrc + voffset into LDS at lds_byte_addr + lane * 4 * VEC.
template <int VEC>
__device__ inline void dma_copy(const u32x4 &rsrc, unsigned voffset, unsigned lds_byte_addr) {
  const u32x4 r = uniform_rsrc(rsrc);
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_byte_addr);
  if constexpr (VEC == 4) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voffset), "s"(r)
                 : "memory");
  } else {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voffset), "s"(r)
                 : "memory");
  }
}

// The same copy with a per-wave byte offset `soffset` (an SGPR) added to the
// address. Only used where no lane's chunk crosses the end of the resource
// range, so the zero fill does not depend on whether the hardware counts
// soffset in its range check: lanes meant to read zeros carry kOutOfRange in
// voffset, every other lane reads inside the matrix.
template <int VEC>
__device__ inline void dma_copy_soff(const u32x4 &rsrc, unsigned voffset, unsigned soffset,
                                     unsigned lds_byte_addr) {
  const u32x4 r = uniform_rsrc(rsrc);
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds_byte_addr);
  const unsigned so = __builtin_amdgcn_readfirstlane(soffset);
  if constexpr (VEC == 4) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(m0), "v"(voffset), "s"(r), "s"(so)
                 : "memory");
  } else {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :
                 : "s"(m0), "v"(voffset), "s"(r), "s"(so)
                 : "memory");
  }
}

template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// f(integral_constant<J>) for J = 0 .. N-1, in order.
template <int J, int N, class F>
__device__ inline void unroll_steps(F &&f) {
  if constexpr (J < N) {
    f(std::integral_constant<int, J>());
    unroll_steps<J + 1, N>(f);
  }
}

// f(integral_constant<R>) for the one R in [R0, RMAX] that equals r (none if
// r is outside).
template <int R0, int RMAX, class F>
__device__ inline void dispatch_count(int r, F &&f) {
  if constexpr (R0 <= RMAX) {
    if (r == R0) f(std::integral_constant<int, R0>());
    else dispatch_count<R0 + 1, RMAX>(r, f);
  }
}

// Swizzle of K-contiguous rows: with 4 chunks per row (BK = 16) 16
// consecutive rows are told apart by r % 4 (bank quarter) and (r / 4) % 4
// (chunk); with 8 chunks per row (BK = 32) by r % 2 and (r / 2) % 8.
template <int CH>
__device__ inline int swz_k(int r) {
  return CH == 4 ? ((r >> 2) & 3) : ((r >> 1) & 7);
}

// One operand of the copy-fed kernel: BX output rows (A: BX = BM) or columns
// (B: BX = BN) by a K step of BK, stored K-contiguous (KMAJOR) or
// M/N-contiguous in global memory, with row stride ld. Per wave: its share of
// the stage's copy instructions and its fragment read offsets.
//
// M/N-contiguous operands are stored in LDS as BK rows of BX floats, the
// 16-column blocks of row k flipped by ((k / KS) % NQ) * MI columns (XOR),
// so the NQ lane groups of a fragment read, which read NQ rows KS apart, hit
// NQ different 16-bank windows. That needs BX to be a power of two. A width
// that is not (BX = 96) is stored as BX / 32 panels of 32 columns instead
// (PANEL), each BK = 32 rows of 32 floats, 16 x 16 blocks only (NQ = 4 lane
// groups, KS = 8): row k = 8q + c of a panel sits in row slot
// 16 (q & 1) + 2c + (q >> 1), its two 16-column halves swapped when q is
// odd. A read by the four lane groups (rows 8q + c, one 16-column half) then
// lands in four different 16-float windows modulo 64 floats (the slot's
// parity and the swap tell them apart) and in two different ones modulo 32
// within each half-wave, so it is free of bank conflicts with 64 banks and
// with 32. A copy fills 8 row slots of one panel.
template <int MI, int BX, int BK, int WX, int NW, bool KMAJOR, int VEC>
struct DmaOperand {
  static constexpr int NQ = 64 / MI;            // lane groups of an instruction
  static constexpr int KS = BK / NQ;            // k per lane group per K step
  static constexpr int NG = KS / 4;             // fragment groups per K step
  static constexpr int F = WX / MI;             // blocks per wave along x
  static constexpr bool PANEL = !KMAJOR && (BX & (BX - 1)) != 0;
  static constexpr int ROW = KMAJOR ? BK : (PANEL ? 32 : BX);   // floats per LDS row
  static constexpr int CH = ROW / 4;            // 16-byte chunks per LDS row
  static constexpr int EP = ROW / VEC;          // lanes per LDS row in one copy
  static constexpr int RP = 64 / EP;            // LDS rows per copy
  static constexpr int I = KMAJOR ? BX / RP : (BX / ROW) * (BK / RP);   // copies per stage
  static constexpr int L = I / NW;              // copies per wave
  static constexpr int COPY_BYTES = 256 * VEC;  // LDS bytes one copy fills
  // LDS floats from fragment row k to row k + 1 (M/N-contiguous operands).
  static constexpr int K_STRIDE = PANEL ? 64 : BX;
  // M/N-contiguous with 4 blocks per wave: block f takes rows (or columns)
  // x = 4*i + f of the wave's range instead of f*MI + i, so a lane's four
  // values at one k are adjacent and one 16-byte read fetches them.
  static constexpr bool INTERLEAVE = !KMAJOR && F == 4;
  static constexpr int NRD = KMAJOR ? NG : (INTERLEAVE ? 1 : F);   // read offsets per lane
  static_assert(VEC == 4 || VEC == 1, "16- or 4-byte copies");
  static_assert(!KMAJOR || CH == 4 || CH == 8, "K step of 16 or 32");
  static_assert(EP <= 64 && 64 % EP == 0, "whole LDS rows per copy");
  static_assert(KMAJOR || PANEL || BX >= NQ * MI, "column flips stay inside a row");
  static_assert(!PANEL || (MI == 16 && BK == 32 && VEC == 4 && BX % 32 == 0 && !INTERLEAVE),
                "panels: 16x16 blocks, K step 32, 16-byte copies, whole panels");
  static_assert(I % NW == 0, "copies split evenly over waves");

  unsigned voff[L];  // lane's byte offset from the tile's first element at step 0
                     // (kOutOfRange when its row or column lies outside the matrix)
  unsigned lds[L];   // byte offset of the copy within the operand's stage region
  int kk[L];         // KMAJOR: first k of the lane's chunk; else: its k row
  bool ok[L];        // row or column inside the matrix
  int rd[NRD];       // fragment read offsets within the operand's stage region (floats)

  __device__ inline void setup(int lane, int wave, int x0, int X, int ld, int q, int li, int wx) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int n = wave + NW * i;          // copy index within the stage
      const int r = n * RP + lane / EP;     // LDS row
      const int pe = (lane % EP) * VEC;     // physical float within the LDS row
      if constexpr (KMAJOR) {
        const int ke = ((pe / 4) ^ swz_k<CH>(r)) * 4 + pe % 4;   // logical k
        ok[i] = x0 + r < X;
        kk[i] = ke;
        voff[i] = ok[i] ? (static_cast<unsigned>(r) * static_cast<unsigned>(ld) + ke) * 4u
                        : kOutOfRange;
      } else if constexpr (PANEL) {
        // Row slot sr of panel n / (BK / RP) holds k row 8 grp + c, grp being
        // the lane group that reads it.
        const int sr = r % BK;
        const int grp = 2 * (sr % 2) + sr / 16;
        const int k = 8 * grp + (sr / 2) % 8;
        const int xe = 32 * (n / (BK / RP)) + (pe ^ (16 * (grp & 1)));
        ok[i] = x0 + xe < X;
        kk[i] = k;
        voff[i] = ok[i] ? (static_cast<unsigned>(k) * static_cast<unsigned>(ld) + xe) * 4u
                        : kOutOfRange;
      } else {
        const int xe = pe ^ (((r / KS) % NQ) * MI);              // logical column
        ok[i] = x0 + xe < X;
        kk[i] = r;
        voff[i] = ok[i] ? (static_cast<unsigned>(r) * static_cast<unsigned>(ld) + xe) * 4u
                        : kOutOfRange;
      }
      lds[i] = static_cast<unsigned>(n * COPY_BYTES);
    }
    // For row x = wx*WX + f*MI + li the swizzle swz_k(x) does not depend on f
    // (f*MI moves x by a multiple of 16 rows), and the columns of lane
    // group q are flipped by q*MI.
#pragma unroll
    for (int j = 0; j < NRD; ++j) {
      if constexpr (KMAJOR) {
        const int x = wx * WX + li;
        rd[j] = x * BK + 4 * (((q * KS + 4 * j) / 4) ^ swz_k<CH>(x));
      } else if constexpr (INTERLEAVE) {
        rd[j] = q * KS * BX + ((wx * WX + 4 * li) ^ (q * MI));
      } else if constexpr (PANEL) {
        // block j's 16 columns lie in one panel; row 8q + c is at slot
        // 16 (q & 1) + (q >> 1) + 2c
        const int x = wx * WX + j * MI + li;
        rd[j] = (x / 32) * (32 * BK) + (16 * (q & 1) + (q >> 1)) * 32 + ((x % 32) ^ (16 * (q & 1)));
      } else {
        rd[j] = q * KS * BX + ((wx * WX + j * MI + li) ^ (q * MI));
      }
    }
  }

  // Reads per fragment group, and read X of load() alone.
  static constexpr int NREADS = KMAJOR ? F : (INTERLEAVE ? 4 : 4 * F);
  __device__ inline void load_part(const float *region, int g, int X, floatx4 (&frag)[F]) const {
    if constexpr (KMAJOR) {
      frag[X] = *reinterpret_cast<const floatx4 *>(region + rd[g] + X * MI * BK);
    } else if constexpr (INTERLEAVE) {
      const floatx4 v = *reinterpret_cast<const floatx4 *>(region + rd[0] + (4 * g + X) * BX);
#pragma unroll
      for (int f = 0; f < F; ++f) frag[f][X] = v[f];
    } else {
      frag[X % F][X / F] = region[rd[X % F] + (4 * g + X / F) * K_STRIDE];
    }
  }

  // Offset, within the wave's x range, of value i of block f.
  __device__ static constexpr int x_of(int f, int i) { return INTERLEAVE ? 4 * i + f : f * MI + i; }

  // Bytes a lane's offset advances per K step.
  __device__ static inline unsigned step_bytes(int ld) {
    return KMAJOR ? 4u * BK : 4u * BK * static_cast<unsigned>(ld);
  }

  // Whether copy i holds data of a K step with kr elements of the range left.
  __device__ inline bool k_valid(int i, int kr) const { return kk[i] < kr; }

  // Fragment group g of a stage region into frag[F] (4 consecutive k each).
  __device__ inline void load(const float *region, int g, floatx4 (&frag)[F]) const {
    if constexpr (KMAJOR) {
#pragma unroll
      for (int f = 0; f < F; ++f)
        frag[f] = *reinterpret_cast<const floatx4 *>(region + rd[g] + f * MI * BK);
    } else if constexpr (INTERLEAVE) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const floatx4 v = *reinterpret_cast<const floatx4 *>(region + rd[0] + (4 * g + j) * BX);
#pragma unroll
        for (int f = 0; f < F; ++f) frag[f][j] = v[f];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int f = 0; f < F; ++f) frag[f][j] = region[rd[f] + (4 * g + j) * K_STRIDE];
    }
  }
};

template <int MI, int BM, int BN, int BK, int WAVES_M, int WAVES_N, int NS, int VEC, bool A_KMAJOR,
          bool B_KMAJOR>
struct DmaShape {
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int NQ = 64 / MI;
  static constexpr int ACC = MI * MI / 64;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int FM = WM / MI, FN = WN / MI;
  static constexpr int KS = BK / NQ;
  static constexpr int NG = KS / 4;
  using OpA = DmaOperand<MI, BM, BK, WM, NWAVES, A_KMAJOR, VEC>;
  using OpB = DmaOperand<MI, BN, BK, WN, NWAVES, B_KMAJOR, VEC>;
  static constexpr int LPW = OpA::L + OpB::L;     // copies per wave per stage
  static constexpr int A_BYTES = BM * BK * 4;
  static constexpr int STAGE_BYTES = (BM * BK + BK * BN) * 4;
  static_assert(KS % 4 == 0 && (NG == 1 || NG % 2 == 0), "fragment groups");
  static_assert(NS >= 3 && NS <= 4, "3 or 4 stages");
  static_assert(NS * STAGE_BYTES <= 160 * 1024, "fits LDS");
  static_assert((NS - 1) * LPW < 64, "vmcnt wait values fit the counter");
  static_assert(NG % 2 == 0 || NS % 2 == 0, "fragment slots repeat with the stage ring");
};

// C <- alpha * op(A) op(B) + beta * C for one output tile (row stride ldc),
// or, for a tile that map_tile splits, the partial product of one K range
// into workspace slab `split` (ws + split * slab, row stride N, written as
// is). op(A) is K-contiguous when A_KMAJOR (A given M x K), op(B) when
// B_KMAJOR (B given N x K, i.e. transposed). beta == 0: C is not read.
//
// The tile order comes as scalars (its whole-tile count, the multipliers of
// its divisors by 8 * tiles_n and by the last group's rows, their two shifts
// packed 8 bits apart, the split count: see kernel_order), and the arguments
// that the tile order and the first copies need come first: the library is
// built with the first 12 arguments (14 dwords, the most there is room for)
// preloaded into scalar registers at wave launch, so the tile order, the
// address set-up and the first copies do not wait for the kernel-argument
// read (about 600 clocks, its first access missing every cache); the others
// arrive meanwhile, needed by the epilogue or on the split path only.
template <int MI, int BM, int BN, int BK, int WAVES_M, int WAVES_N, int NS, int VEC,
          int WAVES_PER_EU, bool A_KMAJOR, bool B_KMAJOR>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WAVES_M * WAVES_N,
                                                      64 * WAVES_M * WAVES_N),
                          amdgpu_waves_per_eu(WAVES_PER_EU, WAVES_PER_EU)))
void mfma_dma_gemm_kernel(const float *__restrict__ A, const float *__restrict__ B, int M, int N,
                          int K, int lda, int ldb, int dp_tiles, unsigned group_mul,
                          unsigned rows_mul, unsigned shifts, int splits, float *__restrict__ C,
                          float *__restrict__ ws, int ldc, float alpha, float beta, int k_chunk,
                          long long slab) {
  using S = DmaShape<MI, BM, BN, BK, WAVES_M, WAVES_N, NS, VEC, A_KMAJOR, B_KMAJOR>;
  using OpA = typename S::OpA;
  using OpB = typename S::OpB;
  using Op = Mfma<MI>;
  using acc_t = typename Op::acc_t;
  constexpr int FM = S::FM, FN = S::FN, NG = S::NG, LPW = S::LPW;
  constexpr int STAGE_F = S::STAGE_BYTES / 4;
  // A wave with more than 4 copies per step (one wave per SIMD, 16 x 16
  // blocks: a 32-clock MFMA is all that covers a stall) interleaves the main
  // loop's fragment reads and copies with its MFMAs one by one (group_spread)
  // instead of issuing them in bursts: the reads of a CU's waves share the
  // LDS and their copies one address unit, so a burst keeps a wave from its
  // next MFMA while it waits for its turn there.
  constexpr bool kSpreadCopies = LPW > 4;

  // The stages, then one float of padding that no copy writes: a real store
  // into it keeps the compiler from treating the array as never written (the
  // copies write it behind the compiler's back), and since no copy lands
  // there it needs no ordering against them.
  __shared__ __attribute__((aligned(16))) float smem[NS * STAGE_F + 4];
  if (threadIdx.x == 0) smem[NS * STAGE_F] = 0.0f;
  // The operand pointers are needed only after the tile arithmetic; asking
  // for them here issues their kernel-argument loads with the others, one
  // round trip instead of two on the way to the first copy.
  asm volatile("" : : "s"(A), "s"(B));

  // The tile coordinates are uniform; readfirstlane says so to the compiler,
  // which otherwise keeps the results of map_tile in vector registers and
  // everything derived from them (the buffer resources, the copy bases) with
  // them.
  TileOrder order;
  order.tiles_m = static_cast<int>((static_cast<unsigned>(M) + BM - 1) / BM);
  order.tiles_n = static_cast<int>((static_cast<unsigned>(N) + BN - 1) / BN);
  order.splits = splits;
  order.dp_tiles = dp_tiles;
  order.per_group = FastDiv{group_mul, shifts & 0xffu};
  order.last_rows = FastDiv{rows_mul, shifts >> 8};
  const TileCoord tc = map_tile_fast(blockIdx.x, order);
  const int m0 = __builtin_amdgcn_readfirstlane(tc.tm) * BM;
  const int n0 = __builtin_amdgcn_readfirstlane(tc.tn) * BN;
  const int split = __builtin_amdgcn_readfirstlane(tc.split);
  const bool whole = __builtin_amdgcn_readfirstlane(tc.whole) != 0;
  // The K range. k_chunk is not preloaded; the empty asm keeps the compiler
  // from computing the split side on every path (as a select), which would
  // make whole tiles wait for the kernel-argument read.
  int k_begin = 0, k_stop = K;   // k_stop: end of the K range
  if (!whole) {
    asm volatile("" ::: "memory");
    k_begin = split * k_chunk;
    k_stop = min(K, k_begin + k_chunk);
  }
  const int nk_all = (k_stop - k_begin + BK - 1) / BK;
  // A ragged last K step of at most 4 elements (K = 513 ends one element into
  // a step) is not staged through LDS: its operands go straight from global
  // memory into registers, loaded early (reg_step_load) and multiplied after
  // the ring's last step (reg_step_mfma). Small register tiles only: those
  // whose last steps are unrolled (a long step hides a stage's cost) and
  // that have room for the 4 * (FM + FN) registers the operands take. The
  // ring then runs the whole steps [k_begin, k_end) only.
  constexpr bool kSmallTile = FM * FN * S::ACC + 8 * (FM + FN) <= 96;
  constexpr bool kRegStep = FM * FN * S::ACC + 12 * (FM + FN) <= 96;
  const int kr_tail = k_stop - (k_begin + (nk_all - 1) * BK);
  const bool reg_step = kRegStep && nk_all >= 2 && kr_tail <= 4;
  const int nk = reg_step ? nk_all - 1 : nk_all;           // steps through the LDS ring
  const int k_end = reg_step ? k_stop - kr_tail : k_stop;  // where those steps end

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int q = lane / MI;
  const int li = lane % MI;
  const unsigned smem_base =
      static_cast<unsigned>(reinterpret_cast<unsigned long long>(
          (__attribute__((address_space(3))) float *)smem));

  OpA opa;
  OpB opb;
  opa.setup(lane, wave, m0, M, lda, q, li, wm);
  opb.setup(lane, wave, n0, N, ldb, q, li, wn);

  // One buffer resource per operand for the whole K range: base at the
  // tile's first element, range ending exactly at the operand's last element,
  // so a chunk running past it reads zeros. Step s adds s times a constant
  // to each lane's offset; the host keeps every valid offset below 2^31, and
  // offsets that start at kOutOfRange stay past the range.
  const long long a_first = A_KMAJOR ? (long long)m0 * lda + k_begin : (long long)k_begin * lda + m0;
  const long long a_end = A_KMAJOR ? (long long)(M - 1) * lda + K : (long long)(K - 1) * lda + M;
  const long long b_first = B_KMAJOR ? (long long)n0 * ldb + k_begin : (long long)k_begin * ldb + n0;
  const long long b_end = B_KMAJOR ? (long long)(N - 1) * ldb + K : (long long)(K - 1) * ldb + N;
  const u32x4 ra = make_buffer_rsrc(A + a_first, 4 * (a_end - a_first));
  const u32x4 rb = make_buffer_rsrc(B + b_first, 4 * (b_end - b_first));
  const unsigned a_step = OpA::step_bytes(lda), b_step = OpB::step_bytes(ldb);
  // Copies of a step whose K range is whole and not the last: no chunk
  // crosses the end of an operand, so the step's advance goes in soffset and
  // the lane offsets stay loop-invariant (no vector add in front of a copy).
  // Copies c0 .. c1-1 of the wave's LPW (A's first, then B's).
  auto issue_full_part = [&](int step, unsigned stage_byte, auto c0_c, auto c1_c) {
    constexpr int C0 = decltype(c0_c)::value, C1 = decltype(c1_c)::value;
    const unsigned da = a_step * step, db = b_step * step;
#pragma unroll
    for (int i = 0; i < OpA::L; ++i)
      if (i >= C0 && i < C1) dma_copy_soff<VEC>(ra, opa.voff[i], da, stage_byte + opa.lds[i]);
#pragma unroll
    for (int i = 0; i < OpB::L; ++i)
      if (OpA::L + i >= C0 && OpA::L + i < C1)
        dma_copy_soff<VEC>(rb, opb.voff[i], db, stage_byte + S::A_BYTES + opb.lds[i]);
  };
  auto issue_full = [&](int step, unsigned stage_byte) {
    issue_full_part(step, stage_byte, std::integral_constant<int, 0>(),
                    std::integral_constant<int, LPW>());
  };
  // Copies of any step: chunks past the end of the K range read zeros
  // (copies c0 .. c1-1 of the wave's LPW, or all).
  auto issue_checked_part = [&](int step, unsigned stage_byte, auto c0_c, auto c1_c) {
    constexpr int C0 = decltype(c0_c)::value, C1 = decltype(c1_c)::value;
    const int kr = k_end - (k_begin + step * BK);   // K elements left in this step
    const unsigned da = a_step * step, db = b_step * step;
#pragma unroll
    for (int i = 0; i < OpA::L; ++i)
      if (i >= C0 && i < C1)
        dma_copy<VEC>(ra, opa.k_valid(i, kr) ? opa.voff[i] + da : kOutOfRange,
                      stage_byte + opa.lds[i]);
#pragma unroll
    for (int i = 0; i < OpB::L; ++i)
      if (OpA::L + i >= C0 && OpA::L + i < C1)
        dma_copy<VEC>(rb, opb.k_valid(i, kr) ? opb.voff[i] + db : kOutOfRange,
                      stage_byte + S::A_BYTES + opb.lds[i]);
  };
  auto issue_checked = [&](int step, unsigned stage_byte) {
    issue_checked_part(step, stage_byte, std::integral_constant<int, 0>(),
                       std::integral_constant<int, LPW>());
  };
  // Wait until this wave's copies of a step have landed while the copies of
  // `later` steps issued after it may stay in flight (vmcnt counts this
  // wave's outstanding loads, oldest first).
  auto wait_landed = [&](int later) {
    if constexpr (NS >= 4) {
      if (later >= 3) { wait_vmcnt<3 * LPW>(); return; }
    }
    if (later >= 2) { wait_vmcnt<2 * LPW>(); return; }
    if (later >= 1) { wait_vmcnt<LPW>(); return; }
    wait_vmcnt<0>();
  };
  auto barrier = [&]() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory"); };
  // When the K range does not end on a 16-byte chunk, the chunk of each
  // K-contiguous row that straddles its end also brought in up to three
  // floats past it (the row's padding or the next row). Once this wave's
  // copies of the last step have landed, it zeroes those floats in the chunks
  // it copied itself.
  auto zero_k_tail = [&](int step) {
    if constexpr (VEC == 4 && (A_KMAJOR || B_KMAJOR)) {
      const int kr = k_end - (k_begin + step * BK);
      if (step != nk - 1 || kr % 4 == 0) return;
      float *stage = smem + (step % NS) * STAGE_F;
      if constexpr (A_KMAJOR) {
#pragma unroll
        for (int i = 0; i < OpA::L; ++i) {
          if (opa.ok[i] && opa.kk[i] < kr && opa.kk[i] + 4 > kr) {
            float *dst = stage + opa.lds[i] / 4 + lane * 4;
            for (int e = kr - opa.kk[i]; e < 4; ++e) dst[e] = 0.0f;
          }
        }
      }
      if constexpr (B_KMAJOR) {
#pragma unroll
        for (int i = 0; i < OpB::L; ++i) {
          if (opb.ok[i] && opb.kk[i] < kr && opb.kk[i] + 4 > kr) {
            float *dst = stage + S::A_BYTES / 4 + opb.lds[i] / 4 + lane * 4;
            for (int e = kr - opb.kk[i]; e < 4; ++e) dst[e] = 0.0f;
          }
        }
      }
    }
  };

  floatx4 fa[2][FM];
  floatx4 fb[2][FN];
  auto load_frags = [&](const float *st, int g, int slot) {
    opa.load(st, g, fa[slot]);
    opb.load(st + S::A_BYTES / 4, g, fb[slot]);
  };

  acc_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < S::ACC; ++v) acc[i][j][v] = 0.0f;
  auto mfma_step = [&](int slot, int j) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        acc[fm][fn] = Op::run(fa[slot][fm][j], fb[slot][fn][j], acc[fm][fn]);
  };

  // The ragged step's operands: instruction s < kr_tail takes k = k_end +
  // q*KS + s in lane group q, real only in group 0 (kr_tail <= 4 <= KS).
  // Raw buffer loads through the copies' ranges, only the kr_tail that are
  // needed per fragment (a uniform count N, dispatched): one lane offset per
  // fragment, kOutOfRange in the lanes that read zero (group q > 0, rows or
  // columns outside the matrix: no memory access), and instruction s's k in
  // the scalar offset. They are issued just before the ring's first copies:
  // issued after them, they would queue behind the CU's prologue copies in
  // the shared address unit (about 430 clocks); issued before, they cost
  // their few instructions and complete before step 0 does (a wave's loads
  // complete in the order issued), so the wait for step 0 covers them; issued
  // in the main loop's first step instead, they missed the L2 and held the
  // next step's wait (the main loop +400 clocks).
  floatx4 ra_reg[FM], rb_reg[FN];
  auto reg_step_load = [&](auto n_c) {
    constexpr int N_LOADS = decltype(n_c)::value;
    // The copies' resources, in the form the load builtin takes: same base,
    // the same range capped one byte lower (every valid element ends well
    // below 2^31).
    auto rsrc = [](const float *base, unsigned range) {
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), static_cast<short>(0),
                                               static_cast<int>(min(range, 0x7fffffffu)), 0x00020000);
    };
    const __amdgpu_buffer_rsrc_t la = rsrc(A + a_first, ra[2]);
    const __amdgpu_buffer_rsrc_t lb = rsrc(B + b_first, rb[2]);
    const unsigned k0 = static_cast<unsigned>(k_end - k_begin);   // k - k_begin of instruction 0
    const int a_k = A_KMAJOR ? 4 : 4 * lda;   // bytes from one k to the next
    const int b_k = B_KMAJOR ? 4 : 4 * ldb;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const unsigned x = static_cast<unsigned>(wm * S::WM + OpA::x_of(fm, li));
      const unsigned off = A_KMAJOR ? x * static_cast<unsigned>(lda) + k0
                                    : k0 * static_cast<unsigned>(lda) + x;
      const int vo = static_cast<int>(q == 0 && m0 + static_cast<int>(x) < M ? 4u * off : kOutOfRange);
#pragma unroll
      for (int e = 0; e < N_LOADS; ++e)
        ra_reg[fm][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(la, vo, e * a_k, 0));
    }
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const unsigned x = static_cast<unsigned>(wn * S::WN + OpB::x_of(fn, li));
      const unsigned off = B_KMAJOR ? x * static_cast<unsigned>(ldb) + k0
                                    : k0 * static_cast<unsigned>(ldb) + x;
      const int vo = static_cast<int>(q == 0 && n0 + static_cast<int>(x) < N ? 4u * off : kOutOfRange);
#pragma unroll
      for (int e = 0; e < N_LOADS; ++e)
        rb_reg[fn][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lb, vo, e * b_k, 0));
    }
  };
  auto reg_step_mfma = [&]() {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (e < kr_tail) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn)
            acc[fm][fn] = Op::run(ra_reg[fm][e], rb_reg[fn][e], acc[fm][fn]);
      }
    }
  };

  // In the last step of the K range only kr_last elements (1 .. BK) are
  // real; instruction s of a step (4 * group + j) takes k = q*KS + s for lane
  // group q, so from s = kr_last on it would only add the zero fill: skipped,
  // and so are fragment reads that only such instructions would use. (A
  // zero-fill product adds +0.0, which leaves an accumulator's bits as they
  // are: it starts at +0.0 and never becomes -0.0.)
  const int kr_last = k_end - (k_begin + (nk - 1) * BK);
  // Whether any instruction of the last step can be skipped: instruction s
  // is needed while s < kr_last, and a step has KS of them. Otherwise the
  // last step runs without the per-instruction branches (they cost ~15
  // clocks each in front of an MFMA).
  const bool skip_some = kr_last < S::KS;

  // One fragment group of the spread schedule (steps before the range's
  // last): its 4 * FM * FN MFMAs (by instruction, then block) from fragment
  // slot `slot`, the reads of the next group's fragments (group rd_g of
  // region rd_st, into slot ^ 1) two after each of the first MFMAs, then
  // (copy mode CM: 1 whole step, 2 range-checked) the LPW copies of step
  // cp_step into stage byte cp_stage one after every third MFMA from the
  // group's second quarter on. The reads end within the group's first
  // quarter, or its first half when both operands are read 4 bytes at a
  // time (M- and N-contiguous panels: 12 reads each at 96 x 96), so the
  // last of them has at least half a group of MFMAs to land.
  constexpr int kNm = 4 * FM * FN;
  constexpr int kNra = OpA::NREADS, kNr = kNra + OpB::NREADS;
  auto group_spread = [&](int slot, const float *rd_st, int rd_g, auto cm_c, int cp_step,
                          unsigned cp_stage) {
    constexpr int CM = decltype(cm_c)::value;
    constexpr int NC = CM ? LPW : 0;
    static_assert(!kSpreadCopies || (kNr <= kNm && kNm / 4 + 3 * LPW <= kNm),
                  "side work fits the group");
    unroll_steps<0, kNm>([&](auto m_c) {
      constexpr int Mi = decltype(m_c)::value;
      constexpr int j = Mi / (FM * FN), fm = (Mi % (FM * FN)) / FN, fn = Mi % FN;
      acc[fm][fn] = Op::run(fa[slot][fm][j], fb[slot][fn][j], acc[fm][fn]);
      __builtin_amdgcn_sched_barrier(0);
      unroll_steps<2 * Mi, 2 * Mi + 2>([&](auto x_c) {
        constexpr int X = decltype(x_c)::value;
        if constexpr (X < kNra) opa.load_part(rd_st, rd_g, X, fa[slot ^ 1]);
        else if constexpr (X < kNr)
          opb.load_part(rd_st + S::A_BYTES / 4, rd_g, X - kNra, fb[slot ^ 1]);
      });
      constexpr int C = (Mi - kNm / 4) / 3;
      if constexpr (Mi >= kNm / 4 && (Mi - kNm / 4) % 3 == 0 && C < NC) {
        if constexpr (CM == 1)
          issue_full_part(cp_step, cp_stage, std::integral_constant<int, C>(),
                          std::integral_constant<int, C + 1>());
        else
          issue_checked_part(cp_step, cp_stage, std::integral_constant<int, C>(),
                             std::integral_constant<int, C + 1>());
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Schedule. One barrier per K step t, in its last fragment group. Every
  // read of step t's stage was issued before it (the fragments of a step are
  // read during the step before it and the step itself), so right after it
  // that stage takes the copies of step t+NS; before it this wave waits until
  // its copies of step t+1 (read from that group on) have landed, leaving
  // steps t+2 .. t+NS-1 in flight.
  //
  // Prologue: all NS stages issued (no range checks when the ring's first
  // NS steps are whole and none is the last), step 0 landed, its first
  // fragments. Issuing every stage up front keeps the later stages' copies in
  // the shadow of step 0's latency (the copies of a CU's waves share one
  // address unit; queued behind the barrier they would hold up the first
  // products).
  if constexpr (kRegStep) {
    if (reg_step) dispatch_count<1, 4>(kr_tail, [&](auto n_c) { reg_step_load(n_c); });
  }
  const bool pro_whole = nk > NS;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const unsigned stage = smem_base + static_cast<unsigned>(s * S::STAGE_BYTES);
    if (pro_whole) issue_full(s, stage);
    else if (s < nk) issue_checked(s, stage);
  }
  wait_landed(min(NS, nk) - min(1, nk));
  zero_k_tail(0);
  barrier();
  load_frags(smem, 0, 0);

  // Steady state: steps whose copy targets are whole, non-final steps. The
  // loop is unrolled over the ring, so stage offsets, fragment slots and
  // wait counts are compile-time constants and no step needs a range check:
  // the only branch is the loop's back edge.
  auto k_step_main = [&](int t, auto stage_c) {
    constexpr int ST = decltype(stage_c)::value;
    const float *st = smem + ST * STAGE_F;
    const float *st_next = smem + ((ST + 1) % NS) * STAGE_F;
    if constexpr (kSpreadCopies) {
      unroll_steps<0, NG>([&](auto g_c) {
        constexpr int G = decltype(g_c)::value;
        constexpr int slot = (ST * NG + G) & 1;
        if constexpr (G < NG - 1) {
          group_spread(slot, st, G + 1, std::integral_constant<int, 0>(), 0, 0u);
        } else {
          wait_vmcnt<(NS - 2) * LPW>();
          barrier();
          __builtin_amdgcn_sched_barrier(0);
          group_spread(slot, st_next, 0, std::integral_constant<int, 1>(), t + NS,
                       smem_base + static_cast<unsigned>(ST * S::STAGE_BYTES));
        }
      });
      return;
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int slot = (ST * NG + g) & 1;
      if (g < NG - 1) {
        mfma_step(slot, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_frags(st, g + 1, slot ^ 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 1; j < 4; ++j) mfma_step(slot, j);
        __builtin_amdgcn_sched_barrier(0);
      } else {
        wait_vmcnt<(NS - 2) * LPW>();
        barrier();
        __builtin_amdgcn_sched_barrier(0);
        mfma_step(slot, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_frags(st_next, 0, slot ^ 1);
        issue_full(t + NS, smem_base + static_cast<unsigned>(ST * S::STAGE_BYTES));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 1; j < 4; ++j) mfma_step(slot, j);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto mfma_k = [&](int slot, int g, int j, bool final_step) {
    if (!final_step || !skip_some || 4 * g + j < kr_last) mfma_step(slot, j);
  };

  // The last R steps of the K range, t0 .. t0+R-1 (t0 a multiple of NS, so
  // step t0+J uses stage J % NS and, when NG is odd, fragment slots of
  // parity J): everything the main loop knows at compile time is known here
  // too, with the checks of the final steps (copies past the K range read
  // zeros; no copies once the last step is issued, no wait after it).
  auto k_step_last = [&](int t0, auto j_c, auto r_c) {
    constexpr int J = decltype(j_c)::value, R = decltype(r_c)::value;
    constexpr int ST = J % NS;
    constexpr bool kMore = J + 1 < R;        // a step follows
    constexpr bool kIssue = J + NS < R;      // step J+NS still to be copied
    // Steps up to min(R-1, J+NS-1) have been issued; step J+1 must land.
    constexpr int kLater = (R - 1 < J + NS - 1 ? R - 1 : J + NS - 1) - (J + 1);
    const float *st = smem + ST * STAGE_F;
    // The final step issues no copies and reads at most its own next group:
    // it takes the plain form below, whose instruction skip branches once per
    // instruction index rather than once per MFMA.
    if constexpr (kSpreadCopies && kMore) {
      unroll_steps<0, NG>([&](auto g_c) {
        constexpr int G = decltype(g_c)::value;
        constexpr int slot = ((J & 1) * NG + G) & 1;
        if constexpr (G < NG - 1) {
          group_spread(slot, st, G + 1, std::integral_constant<int, 0>(), 0, 0u);
        } else {
          wait_vmcnt<kLater * LPW>();
          if constexpr (J + 2 == R) zero_k_tail(t0 + J + 1);
          barrier();
          __builtin_amdgcn_sched_barrier(0);
          constexpr int kMode = !kIssue ? 0 : (J + NS < R - 1 ? 1 : 2);
          group_spread(slot, smem + ((ST + 1) % NS) * STAGE_F, 0,
                       std::integral_constant<int, kMode>(), t0 + J + NS,
                       smem_base + static_cast<unsigned>(ST * S::STAGE_BYTES));
        }
      });
      return;
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int slot = ((J & 1) * NG + g) & 1;
      if (g < NG - 1) {
        mfma_k(slot, g, 0, !kMore);
        __builtin_amdgcn_sched_barrier(0);
        if (kMore || 4 * (g + 1) < kr_last) load_frags(st, g + 1, slot ^ 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 1; j < 4; ++j) mfma_k(slot, g, j, !kMore);
        __builtin_amdgcn_sched_barrier(0);
      } else {
        if constexpr (kMore) {
          wait_vmcnt<kLater * LPW>();
          if constexpr (J + 2 == R) zero_k_tail(t0 + J + 1);
          barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_k(slot, g, 0, !kMore);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kMore) load_frags(smem + ((ST + 1) % NS) * STAGE_F, 0, slot ^ 1);
        // A copy of a step before the last is of a whole step, as in the
        // main loop (the advance in soffset, no checks); only the last
        // step's copies need the range checks.
        if constexpr (kIssue && J + NS < R - 1)
          issue_full(t0 + J + NS, smem_base + static_cast<unsigned>(ST * S::STAGE_BYTES));
        else if constexpr (kIssue)
          issue_checked(t0 + J + NS, smem_base + static_cast<unsigned>(ST * S::STAGE_BYTES));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 1; j < 4; ++j) mfma_k(slot, g, j, !kMore);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Any one of the last steps, with run-time stage, slot parity P, waits and
  // checks (kernels with many accumulators: see below).
  auto k_step_tail = [&](int t, auto parity) {
    constexpr int P = decltype(parity)::value;
    const bool more = t + 1 < nk;
    const float *st = smem + (t % NS) * STAGE_F;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int slot = (P * NG + g) & 1;
      if (g < NG - 1) {
        mfma_k(slot, g, 0, !more);
        __builtin_amdgcn_sched_barrier(0);
        if (more || 4 * (g + 1) < kr_last) load_frags(st, g + 1, slot ^ 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 1; j < 4; ++j) mfma_k(slot, g, j, !more);
        __builtin_amdgcn_sched_barrier(0);
      } else {
        // Steps up to min(nk-1, t+NS-1) have been issued; step t+1 must
        // have landed.
        if (more) {
          wait_landed(min(nk - 1, t + NS - 1) - (t + 1));
          zero_k_tail(t + 1);
          barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
        mfma_k(slot, g, 0, !more);
        __builtin_amdgcn_sched_barrier(0);
        if (more) load_frags(smem + ((t + 1) % NS) * STAGE_F, 0, slot ^ 1);
        if (t + NS < nk)
          issue_checked(t + NS, smem_base + static_cast<unsigned>(((t + NS) % NS) * S::STAGE_BYTES));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 1; j < 4; ++j) mfma_k(slot, g, j, !more);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // A main-loop pass covers steps t .. t+NS-1 and copies steps up to
  // t+2*NS-1, which must all be whole and before the last step nk-1.
  const int n_main = nk >= 2 * NS + 1 ? (nk - 2 * NS - 1) / NS + 1 : 0;
  int t = 0;
  for (int it = 0; it < n_main; ++it, t += NS) {
    k_step_main(t, std::integral_constant<int, 0>());
    k_step_main(t + 1, std::integral_constant<int, 1>());
    k_step_main(t + 2, std::integral_constant<int, 2>());
    if constexpr (NS >= 4) k_step_main(t + 3, std::integral_constant<int, 3>());
  }
  // nk - t steps are left: NS+1 .. 2*NS after main-loop passes, nk (at most
  // 2*NS) without any. t is a multiple of NS, hence even when NG is odd (NS
  // is then even). A K step of a small register tile is short (512 clocks
  // for one 32x32 block per wave), and the run-time stage arithmetic and
  // branches of the looped form cost ~300 clocks of it, so such tiles get one
  // unrolled copy of the last steps per count. With many accumulators the
  // 2*NS copies make the register allocator spill them, and a long K step
  // hides the looped form's cost, so those keep the loop.
  constexpr bool kUnrolledTail = kSmallTile;
  if constexpr (kUnrolledTail) {
    dispatch_count<1, 2 * NS>(nk - t, [&](auto r_c) {
      unroll_steps<0, decltype(r_c)::value>([&](auto j_c) { k_step_last(t, j_c, r_c); });
    });
    if (reg_step) reg_step_mfma();
  } else {
    for (; t < nk; t += 2) {
      k_step_tail(t, std::integral_constant<int, 0>());
      if (t + 1 < nk) k_step_tail(t + 1, std::integral_constant<int, 1>());
    }
  }

  // k_chunk stays live until here: were its register reused after the split
  // path's last read, the reuse would have to wait for the argument read
  // that fills it, on every path.
  asm volatile("" : : "s"(k_chunk));
  // Output of this workgroup: C, or its K range's workspace slab (the
  // arguments that say so are not among the preloaded ones: read here, not
  // before the first copies).
  float *__restrict__ Cout = whole ? C : ws + (long long)split * slab;
  const int ldo = whole ? ldc : N;
  const float alpha_o = whole ? alpha : 1.0f;
  const float beta_o = whole ? beta : 0.0f;

  // Epilogue: accumulator v of block (fm, fn) is output row Op::row(q, v) and
  // column li of that block. With beta != 0 the C values of a block row are
  // all loaded before any is used, so their latencies overlap. store_tile
  // (for outputs whose rows are too far apart for the buffer form below):
  // the branches on beta and on whether the tile lies wholly inside C are
  // uniform and taken once; interior tiles store without per-element checks.
  auto store_tile = [&](auto beta_is_zero, auto checked) {
    constexpr bool kBetaZero = decltype(beta_is_zero)::value;
    constexpr bool kChecked = decltype(checked)::value;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      float cv[FN][S::ACC];
      if constexpr (!kBetaZero) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
          const int col = n0 + wn * S::WN + OpB::x_of(fn, li);
#pragma unroll
          for (int v = 0; v < S::ACC; ++v) {
            const int row = m0 + wm * S::WM + OpA::x_of(fm, Op::row(q, v));
            const bool in = !kChecked || (row < M && col < N);
            cv[fn][v] = in ? Cout[(long long)row * ldo + col] : 0.0f;
          }
        }
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int col = n0 + wn * S::WN + OpB::x_of(fn, li);
#pragma unroll
        for (int v = 0; v < S::ACC; ++v) {
          const int row = m0 + wm * S::WM + OpA::x_of(fm, Op::row(q, v));
          if (!kChecked || (row < M && col < N)) {
            float *p = Cout + (long long)row * ldo + col;
            if constexpr (kBetaZero)
              *p = alpha_o * acc[fm][fn][v];
            else
              *p = __builtin_fmaf(alpha_o, acc[fm][fn][v], beta_o * cv[fn][v]);
          }
        }
      }
    }
  };
  // Edge tiles: the same stores through a buffer resource over the output,
  // from the tile's first element to the last element of C (or of the slab):
  // the hardware drops a store whose offset lies past the range (and a load
  // there reads 0), which is where every row at or below M lands, since
  // offsets grow by ldo >= N per row; lanes whose column lies at or past N
  // carry kOutOfRange. Straight-line code, without the branch per element of
  // the checked store_tile (per-wave timestamps on 1001 x 513 x 777: the
  // slowest edge tile's store 2,148 -> 1,788 clocks). Interior tiles keep
  // store_tile, whose first store issues sooner (1,072 against 1,440 clocks
  // for this form). Needs the tile's offsets to fit in 31 bits (BM rows of
  // ldo floats).
  auto store_tile_buffer = [&](auto beta_is_zero) {
    constexpr bool kBetaZero = decltype(beta_is_zero)::value;
    const long long first = (long long)m0 * ldo + n0;
    const long long range = 4 * ((long long)(M - 1) * ldo + N - first);
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        Cout + first, static_cast<short>(0),
        static_cast<int>(range < 0x7fffffffLL ? range : 0x7fffffffLL), 0x00020000);
    unsigned col_off[FN];
    bool col_ok[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int col = wn * S::WN + OpB::x_of(fn, li);
      col_ok[fn] = n0 + col < N;
      col_off[fn] = 4u * static_cast<unsigned>(col);
    }
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      unsigned off[FN][S::ACC];
#pragma unroll
      for (int v = 0; v < S::ACC; ++v) {
        const unsigned row_off =
            4u * static_cast<unsigned>(wm * S::WM + OpA::x_of(fm, Op::row(q, v))) *
            static_cast<unsigned>(ldo);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) off[fn][v] = col_ok[fn] ? row_off + col_off[fn] : kOutOfRange;
      }
      float cv[FN][S::ACC];
      if constexpr (!kBetaZero) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int v = 0; v < S::ACC; ++v)
            cv[fn][v] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(rc, static_cast<int>(off[fn][v]), 0, 0));
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
        for (int v = 0; v < S::ACC; ++v) {
          float r;
          if constexpr (kBetaZero)
            r = alpha_o * acc[fm][fn][v];
          else
            r = __builtin_fmaf(alpha_o, acc[fm][fn][v], beta_o * cv[fn][v]);
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, r), rc,
                                                static_cast<int>(off[fn][v]), 0, 0);
        }
      }
    }
  };
  const bool interior = m0 + BM <= M && n0 + BN <= N;
  if (!interior && ((long long)BM * ldo + BN) * 4 < (1LL << 31)) {
    if (beta_o == 0.0f) store_tile_buffer(std::true_type());
    else store_tile_buffer(std::false_type());
    return;
  }
  if (beta_o == 0.0f) {
    if (interior) store_tile(std::true_type(), std::false_type());
    else store_tile(std::true_type(), std::true_type());
  } else {
    if (interior) store_tile(std::false_type(), std::false_type());
    else store_tile(std::false_type(), std::true_type());
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

  const TileCoord tc = map_tile(blockIdx.x, tiles_m, tiles_n, splits, kGroupM);
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
// Sum over the `splits` slabs (`stride` floats apart) at offset `at`, in
// ascending slab order ((w0 + w1) + w2) + ...; the loads of up to 8 slabs are
// issued before their adds, so their latencies overlap instead of adding up.
template <int V>
struct SlabSum;

template <>
struct SlabSum<4> {
  static __device__ inline floatx4 load(const float *p) {
    return *reinterpret_cast<const floatx4 *>(p);
  }
  static __device__ inline floatx4 sum(const float *__restrict__ ws, long long stride,
                                       long long at, int splits) {
    constexpr int kBatch = 8;
    floatx4 s = load(ws + at);
    int p = 1;
    for (; p + kBatch <= splits; p += kBatch) {
      floatx4 v[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) v[b] = load(ws + (long long)(p + b) * stride + at);
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        s[0] = s[0] + v[b][0]; s[1] = s[1] + v[b][1]; s[2] = s[2] + v[b][2]; s[3] = s[3] + v[b][3];
      }
    }
    for (; p < splits; ++p) {
      const floatx4 v = load(ws + (long long)p * stride + at);
      s[0] = s[0] + v[0]; s[1] = s[1] + v[1]; s[2] = s[2] + v[2]; s[3] = s[3] + v[3];
    }
    return s;
  }
};

template <>
struct SlabSum<1> {
  static __device__ inline float sum(const float *__restrict__ ws, long long stride, long long at,
                                     int splits) {
    constexpr int kBatch = 8;
    float s = ws[at];
    int p = 1;
    for (; p + kBatch <= splits; p += kBatch) {
      float v[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) v[b] = ws[(long long)(p + b) * stride + at];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) s = s + v[b];
    }
    for (; p < splits; ++p) s = s + ws[(long long)p * stride + at];
    return s;
  }
};

// Split-K reduction: sum_s ws[s][e] in ascending slab order (so the result
// does not depend on which workgroup finished first), then
// C <- alpha * sum + beta * C (C not read when beta == 0). The slabs are
// dense M x N; C has row stride ldc. V = 4: four consecutive columns per
// lane (N and ldc multiples of 4, 16-byte aligned). Pure streaming:
// S*M*N reads and M*N writes (plus M*N reads when beta != 0), HBM bound.
template <int V>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads)))
void splitk_reduce_kernel(const float *__restrict__ ws, float *__restrict__ C, long long count,
                          int N, int ldc, int splits, float alpha, float beta) {
  const long long stride = (long long)gridDim.x * kThreads;
  const bool dense = ldc == N;
  for (long long e = (long long)blockIdx.x * kThreads + threadIdx.x; e * V < count; e += stride) {
    const long long first = e * V;
    float *out = dense ? C + first : C + (first / N) * ldc + first % N;
    if constexpr (V == 4) {
      const floatx4 s = SlabSum<4>::sum(ws, count, first, splits);
      floatx4 r;
      if (beta == 0.0f) {
        r[0] = alpha * s[0]; r[1] = alpha * s[1]; r[2] = alpha * s[2]; r[3] = alpha * s[3];
      } else {
        const floatx4 c = *reinterpret_cast<const floatx4 *>(out);
        r[0] = __builtin_fmaf(alpha, s[0], beta * c[0]);
        r[1] = __builtin_fmaf(alpha, s[1], beta * c[1]);
        r[2] = __builtin_fmaf(alpha, s[2], beta * c[2]);
        r[3] = __builtin_fmaf(alpha, s[3], beta * c[3]);
      }
      *reinterpret_cast<floatx4 *>(out) = r;
    } else {
      const float s = SlabSum<1>::sum(ws, count, first, splits);
      *out = beta == 0.0f ? alpha * s : __builtin_fmaf(alpha, s, beta * *out);
    }
  }
}

// Reduction of a split tail: for each tile after the first dp_tiles of the
// tile order (map_tile_fast), C <- alpha * sum_s ws[s] + beta * C over its
// elements inside C, the slabs summed in ascending order as above. The slabs
// are M x N with row stride N; only these tiles' elements are read. Grid:
// x = tail tile, y = parts of one tile. V = 4 as above (N and ldc multiples
// of 4, 16-byte aligned: a tile's row segment is then whole float4s).
template <int V>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads)))
void tail_reduce_kernel(const float *__restrict__ ws, float *__restrict__ C, int M, int N, int ldc,
                        TileOrder order, int bm, int bn, float alpha, float beta) {
  const int splits = order.splits;
  int tm, tn;
  grouped_tile_fast(order.dp_tiles + blockIdx.x, order, &tm, &tn);
  const int m0 = tm * bm, n0 = tn * bn;
  const int rows = min(bm, M - m0), cols = min(bn, N - n0);
  const int per_row = (cols + V - 1) / V;
  const int items = rows * per_row;
  const long long slab = (long long)M * N;
  for (int e = blockIdx.y * kThreads + threadIdx.x; e < items; e += gridDim.y * kThreads) {
    const int r = e / per_row;
    const int c = (e - r * per_row) * V;
    const long long w = (long long)(m0 + r) * N + n0 + c;
    float *out = C + (long long)(m0 + r) * ldc + n0 + c;
    if constexpr (V == 4) {
      const floatx4 s = SlabSum<4>::sum(ws, slab, w, splits);
      floatx4 o;
      if (beta == 0.0f) {
        o[0] = alpha * s[0]; o[1] = alpha * s[1]; o[2] = alpha * s[2]; o[3] = alpha * s[3];
      } else {
        const floatx4 cv = *reinterpret_cast<const floatx4 *>(out);
        o[0] = __builtin_fmaf(alpha, s[0], beta * cv[0]);
        o[1] = __builtin_fmaf(alpha, s[1], beta * cv[1]);
        o[2] = __builtin_fmaf(alpha, s[2], beta * cv[2]);
        o[3] = __builtin_fmaf(alpha, s[3], beta * cv[3]);
      }
      *reinterpret_cast<floatx4 *>(out) = o;
    } else {
      const float s = SlabSum<1>::sum(ws, slab, w, splits);
      *out = beta == 0.0f ? alpha * s : __builtin_fmaf(alpha, s, beta * *out);
    }
  }
}

// C <- beta * C over M x N with row stride ldc, +0.0 when beta == 0 (C then
// not read): the whole result when K = 0 or alpha = 0.
// (static: not a template, and the header is compiled in two translation
// units; only gemm_api.hip launches it)
static __global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), unused))
void scale_c_kernel(float *__restrict__ C, long long count, int N, int ldc, float beta) {
  const long long stride = (long long)gridDim.x * kThreads;
  for (long long e = (long long)blockIdx.x * kThreads + threadIdx.x; e < count; e += stride) {
    float *out = ldc == N ? C + e : C + (e / N) * ldc + e % N;
    *out = beta == 0.0f ? 0.0f : beta * *out;
  }
}

}  // namespace gemm

// The optimisation ladder of the yekq.top LeetGPU matrix-multiplication
// walkthrough (sections v0 to v3), rebuilt for 64-lane waves so that each
// step of it can be timed and counted on MI355X next to the matrix-core
// kernels. They exist for that comparison; the planner never picks them.
//
// Every kernel: 256 lanes per workgroup viewed as 16 x 16 (tx = lane % 16,
// ty = lane / 16, so one wave covers tx 0..15 for four consecutive ty), one
// output tile per workgroup, the K range [k_begin, k_end) of split `split`,
// FP32 multiply-add in ascending k, out-of-range outputs never stored.
//   v0: one output per lane, tx along the rows of C: a wave touches 16 rows
//       of A (stride K) and 4 columns of B per k -- the uncoalesced mapping
//       the walkthrough starts from;
//   v1: one output per lane, tx along the columns: 16 consecutive floats of
//       a B row per k, A values shared by 16 lanes;
//   v2: 16 x 16 tiles of A and B staged in LDS per 16-wide K phase, zero
//       filled past the edges, two barriers per phase (the tiling the
//       euler0525 post and hpc.payai.win lesson 10 also teach);
//   v3: each lane computes 4 consecutive outputs of one row (register
//       coarsening along N), 16 x 64 output tile, 16-wide K phases in LDS;
//       v2 is the same kernel with one output per lane.
// The walkthrough's v4 (a 2-D register tile per lane) is valu_gemm_kernel in
// gemm_kernels.hpp.
#pragma once

#include <hip/hip_runtime.h>

namespace gemm {

struct LadderTile {
  int tm, tn, split;
};

// Workgroup id -> tile, in plain order (no XCD awareness, as on the pages):
// K ranges slowest; ROWS_FAST puts consecutive ids on consecutive tile rows.
template <bool ROWS_FAST>
__device__ inline LadderTile ladder_tile(int bid, int tiles_m, int tiles_n) {
  const int tiles = tiles_m * tiles_n;
  LadderTile c;
  c.split = bid / tiles;
  const int t = bid - c.split * tiles;
  if (ROWS_FAST) {
    c.tm = t % tiles_m;
    c.tn = t / tiles_m;
  } else {
    c.tn = t % tiles_n;
    c.tm = t / tiles_n;
  }
  return c;
}

// v0 (ROWS_ALONG_LANES = true) and v1 (false): 16 x 16 outputs per workgroup.
template <bool ROWS_ALONG_LANES>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void ladder_naive_kernel(const float *__restrict__ A, const float *__restrict__ B,
                         float *__restrict__ C, int M, int N, int K, int k_chunk, int tiles_m,
                         int tiles_n, int splits, long long slab) {
  (void)splits;
  const LadderTile tc = ladder_tile<ROWS_ALONG_LANES>(blockIdx.x, tiles_m, tiles_n);
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const int row = tc.tm * 16 + (ROWS_ALONG_LANES ? tx : ty);
  const int col = tc.tn * 16 + (ROWS_ALONG_LANES ? ty : tx);
  if (row >= M || col >= N) return;   // no barriers in this kernel
  const int k_begin = tc.split * k_chunk;
  const int k_end = min(K, k_begin + k_chunk);
  const float *a = A + (long long)row * K;
  const float *b = B + col;
  float sum = 0.0f;
  for (int k = k_begin; k < k_end; ++k) sum += a[k] * b[(long long)k * N];
  C[(long long)tc.split * slab + (long long)row * N + col] = sum;
}

// v2 (TN = 1) and v3 (TN = 4): 16 x (16 * TN) outputs per workgroup; lane
// (tx, ty) computes row ty, columns TN*tx .. TN*tx+TN-1 (v2: one output per
// lane, v3: register coarsening along N). Per K phase of 16 the A tile
// (16 x 16) takes one load per lane and the B tile (16 x 16*TN) TN loads,
// lanes along its rows (coalesced); both are zero filled past the edges of
// the K range and of A and B, and every lane reaches both barriers of the
// phase (hpc.payai.win lesson 10, sections 2 and 3: the write of the tiles is
// published by the first, their reuse is held off by the second).
template <int TN>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void ladder_lds_kernel(const float *__restrict__ A, const float *__restrict__ B,
                       float *__restrict__ C, int M, int N, int K, int k_chunk, int tiles_m,
                       int tiles_n, int splits, long long slab) {
  (void)splits;
  static_assert(TN == 1 || TN == 4, "v2 or v3");
  constexpr int BN = 16 * TN;
  __shared__ float As[16][16];
  __shared__ __attribute__((aligned(16))) float Bs[16][BN];
  const LadderTile tc = ladder_tile<false>(blockIdx.x, tiles_m, tiles_n);
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const int row = tc.tm * 16 + ty;
  const int col0 = tc.tn * BN + TN * tx;
  const int k_begin = tc.split * k_chunk;
  const int k_end = min(K, k_begin + k_chunk);
  float acc[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) acc[j] = 0.0f;
  for (int k0 = k_begin; k0 < k_end; k0 += 16) {
    const int ka = k0 + tx;
    As[ty][tx] = (row < M && ka < k_end) ? A[(long long)row * K + ka] : 0.0f;
    // B tile: element e = j*256 + lane, row e / BN, column e % BN.
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int e = j * 256 + threadIdx.x;
      const int kb = k0 + e / BN, cb = tc.tn * BN + e % BN;
      Bs[e / BN][e % BN] = (kb < k_end && cb < N) ? B[(long long)kb * N + cb] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float a = As[ty][k];
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[j] += a * Bs[k][TN * tx + j];
    }
    __syncthreads();
  }
  if (row < M) {
    float *out = C + (long long)tc.split * slab + (long long)row * N;
#pragma unroll
    for (int j = 0; j < TN; ++j)
      if (col0 + j < N) out[col0 + j] = acc[j];
  }
}

}  // namespace gemm

/*
 * CPU oracle for the row-major FP32 matrix product C = A x B.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or
 * call this file: only the test suite, the smoke check and the bench's CPU
 * baseline leg use it. It shares no code, header, table or helper with the
 * HIP library it checks.
 *
 * What it computes (the plain definition, reached exactly up to one final
 * rounding):
 *
 *   C[i][j] = fl32( sum_{k=0}^{K-1} (double)A[i][k] * (double)B[k][j] )
 *
 * with A an M x K, B a K x N and C an M x N matrix, each dense and
 * row-major (element (r, c) of an R x S matrix sits at r*S + c). This is the
 * element-wise dot-product definition given in the problem statement of the
 * yekq.top LeetGPU "matrix multiplication" walkthrough (section on the
 * problem, the equation for C_{row,col}) and in section 1 of the
 * hpc.payai.win lesson 10 "shared-memory tiled GEMM"; the
 * blog.euler0525.cn post (section "naive implementation") states the same sum
 * with the letters N and K swapped, which this file does not follow.
 *
 * Readings fixed here where the pages are silent:
 *   - accumulation is in IEEE double, over ascending k, starting from +0.0;
 *     an FP32 x FP32 product is exact in double (24+24 <= 53 significand
 *     bits), so only the additions round;
 *   - the double sum is rounded once to FP32 (round to nearest even, the C
 *     conversion);
 *   - alpha = 1, beta = 0: C is overwritten, its prior contents are unused;
 *   - K = 0 gives the empty sum, C = +0.0.
 *
 * Alongside C the oracle returns S[i][j] = sum_k |A[i][k] * B[k][j]| (double),
 * the scale that the per-element acceptance bound |C - ref| <= 1e-5*S + 1e-6
 * is written against.
 *
 * oracle_gemm_i64 is the exact integer product for integer-valued inputs;
 * it is used for the small-integer cases whose every partial sum is exactly
 * representable in FP32.
 *
 * Loop order is i -> k -> j with a double row accumulator of length N, so
 * every C element is still summed in ascending k (bit-identical to the
 * i -> j -> k triple loop) while the j loop runs over contiguous memory.
 * Rows are split across OpenMP threads; each row is computed by one thread
 * only, so the result does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <omp.h>

/* Return value convention: 0 = ok, -1 = bad argument, -2 = out of memory. */

int oracle_num_threads(void) { return omp_get_max_threads(); }

int oracle_gemm_f32(const float *A, const float *B, float *C, double *S,
                    int64_t M, int64_t N, int64_t K, int threads) {
  if (M < 0 || N < 0 || K < 0) return -1;
  if (M == 0 || N == 0) return 0;
  if ((K > 0 && (!A || !B)) || !C) return -1;
  if (threads <= 0) threads = omp_get_max_threads();
  int failed = 0;
#pragma omp parallel num_threads(threads) reduction(| : failed)
  {
    double *acc = (double *)malloc(sizeof(double) * (size_t)N);
    double *sab = (double *)malloc(sizeof(double) * (size_t)N);
    if (!acc || !sab) {
      failed = 1;
    } else {
#pragma omp for schedule(static)
      for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
          acc[j] = 0.0;
          sab[j] = 0.0;
        }
        for (int64_t k = 0; k < K; ++k) {
          const double a = (double)A[i * K + k];
          const float *brow = B + k * N;
          for (int64_t j = 0; j < N; ++j) {
            const double p = a * (double)brow[j];
            acc[j] += p;
            sab[j] += fabs(p);
          }
        }
        for (int64_t j = 0; j < N; ++j) {
          C[i * N + j] = (float)acc[j];
          if (S) S[i * N + j] = sab[j];
        }
      }
    }
    free(acc);
    free(sab);
  }
  return failed ? -2 : 0;
}

/*
 * The same definition evaluated only at the listed (rows[t], cols[t]) pairs,
 * one dot product at a time, in ascending k. Used where the full product is
 * too large to form on the host: every sampled entry is bit-identical to the
 * one oracle_gemm_f32 would produce.
 */
int oracle_gemm_f32_entries(const float *A, const float *B, int64_t M,
                            int64_t N, int64_t K, const int64_t *rows,
                            const int64_t *cols, int64_t count, float *out,
                            double *S, int threads) {
  if (M < 0 || N < 0 || K < 0 || count < 0) return -1;
  if (count == 0) return 0;
  if (!rows || !cols || !out || (K > 0 && (!A || !B))) return -1;
  for (int64_t t = 0; t < count; ++t)
    if (rows[t] < 0 || rows[t] >= M || cols[t] < 0 || cols[t] >= N) return -1;
  if (threads <= 0) threads = omp_get_max_threads();
#pragma omp parallel for num_threads(threads) schedule(dynamic, 16)
  for (int64_t t = 0; t < count; ++t) {
    const int64_t i = rows[t], j = cols[t];
    double acc = 0.0, sab = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const double p = (double)A[i * K + k] * (double)B[k * N + j];
      acc += p;
      sab += fabs(p);
    }
    out[t] = (float)acc;
    if (S) S[t] = sab;
  }
  return 0;
}

/*
 * General form, in the shape of the BLAS SGEMM call that the LeetGPU
 * walkthrough's cuBLAS reference section makes, for row-major storage:
 *
 *   C[i][j] <- alpha * sum_{k=0}^{K-1} opA(i, k) * opB(k, j) + beta * C[i][j]
 *
 *   opA(i, k) = A[i*lda + k]           (trans_a == 0: A stored M x K)
 *             = A[k*lda + i]           (trans_a != 0: A stored K x M, i.e. A^T)
 *   opB(k, j) = B[k*ldb + j]           (trans_b == 0: B stored K x N)
 *             = B[j*ldb + k]           (trans_b != 0: B stored N x K)
 *   element (i, j) of C at C[i*ldc + j].
 *
 * The pages fix alpha = 1, beta = 0 and dense storage (the plain function
 * above); the general form takes the BLAS conventions, read as:
 *   - the sum is the plain function's: FP64, ascending k, from +0.0;
 *   - alpha * sum + beta * c is formed in double (c the FP32 value held in C)
 *     and rounded once to FP32;
 *   - beta == 0: C is not read (NaN or garbage in C does not matter) and the
 *     result is alpha * sum;
 *   - alpha == 0 or K == 0: A and B are not read and the result is beta * c,
 *     or +0.0 when beta == 0;
 *   - only the M x N elements are written; the rest of each C row (up to
 *     ldc) is left as it was.
 * S (dense M x N, may be null) receives |alpha| * sum_k |opA * opB| + |beta * c|,
 * the scale of the acceptance bound.
 */
int oracle_gemm_f32_general(int trans_a, int trans_b, int64_t M, int64_t N,
                            int64_t K, float alpha, const float *A,
                            int64_t lda, const float *B, int64_t ldb,
                            float beta, float *C, int64_t ldc, double *S,
                            int threads) {
  if (M < 0 || N < 0 || K < 0) return -1;
  if (M == 0 || N == 0) return 0;
  const int use_ab = alpha != 0.0f && K > 0;
  if (!C || ldc < N) return -1;
  if (use_ab && (!A || !B)) return -1;
  if (use_ab && lda < (trans_a ? M : K)) return -1;
  if (use_ab && ldb < (trans_b ? K : N)) return -1;
  if (threads <= 0) threads = omp_get_max_threads();
#pragma omp parallel for num_threads(threads) schedule(static)
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t j = 0; j < N; ++j) {
      double sum = 0.0, sab = 0.0;
      if (use_ab) {
        for (int64_t k = 0; k < K; ++k) {
          const double a = trans_a ? (double)A[k * lda + i] : (double)A[i * lda + k];
          const double b = trans_b ? (double)B[j * ldb + k] : (double)B[k * ldb + j];
          sum += a * b;
          sab += fabs(a * b);
        }
      }
      const double c = beta != 0.0f ? (double)C[i * ldc + j] : 0.0;
      double r;
      if (!use_ab)
        r = beta != 0.0f ? (double)beta * c : 0.0;
      else if (beta == 0.0f)
        r = (double)alpha * sum;
      else
        r = (double)alpha * sum + (double)beta * c;
      C[i * ldc + j] = (float)r;
      if (S) S[i * N + j] = fabs((double)alpha) * sab + fabs((double)beta * c);
    }
  }
  return 0;
}

/*
 * Exact integer product: C[i][j] = sum_k A[i][k] * B[k][j] in int64.
 * Exact as long as no partial sum leaves the int64 range; the callers keep
 * |A|, |B| <= 16 and K <= 2^17, far inside it.
 */
int oracle_gemm_i64(const int64_t *A, const int64_t *B, int64_t *C, int64_t M,
                    int64_t N, int64_t K, int threads) {
  if (M < 0 || N < 0 || K < 0) return -1;
  if (M == 0 || N == 0) return 0;
  if ((K > 0 && (!A || !B)) || !C) return -1;
  if (threads <= 0) threads = omp_get_max_threads();
#pragma omp parallel for num_threads(threads) schedule(static)
  for (int64_t i = 0; i < M; ++i) {
    int64_t *crow = C + i * N;
    for (int64_t j = 0; j < N; ++j) crow[j] = 0;
    for (int64_t k = 0; k < K; ++k) {
      const int64_t a = A[i * K + k];
      const int64_t *brow = B + k * N;
      for (int64_t j = 0; j < N; ++j) crow[j] += a * brow[j];
    }
  }
  return 0;
}

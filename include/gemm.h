/*
 * libgemm: row-major FP32 matrix product C = A x B on AMD Instinct MI355X (gfx950).
 *
 * The operation (yekq.top LeetGPU "matrix multiplication" walkthrough, the
 * problem-statement and input/output sections; hpc.payai.win lesson 10
 * "shared-memory tiled GEMM", section 1):
 *
 *   A is M x K, B is K x N, C is M x N, all dense, row-major FP32 in device
 *   memory (element (r, c) of an R x S matrix sits at r*S + c, so the leading
 *   dimensions are K, N and N). Every output is the length-K dot product
 *   C[row][col] = sum_k A[row][k] * B[k][col].
 *
 * C is overwritten (alpha = 1, beta = 0); its prior contents are never read.
 * K = 0 stores +0.0 into all of C (the empty sum). M = 0 or N = 0 does
 * nothing. The sum is evaluated in FP32 (FP32 MFMA products and accumulation;
 * with split-K, S partial sums over contiguous K ranges are added in
 * ascending range order), so results are reproducible run to run for a given
 * plan but are not in general bit-identical to a sequential sum. Whether a
 * given output is split depends on the plan alone (never on timing).
 *
 * Calling convention shared by every entry point:
 *   - Pointers are device pointers on the current HIP device; `stream` is a
 *     HIP stream of that device (0 = the null stream). The work is enqueued
 *     on `stream` and the call returns without synchronising: C is valid once
 *     the stream reaches the end of the enqueued work.
 *   - The caller owns A, B, C and any workspace, and keeps them alive and
 *     unmodified until the stream has passed the work.
 *   - A, B and C are `restrict`: C's bytes must not overlap A's or B's
 *     (A and B may overlap each other). Pointers the call does not access
 *     (all three when M or N is 0, A and B when K is 0) may be null.
 *   - Errors are reported only through the returned status; nothing is
 *     printed and nothing is thrown. Argument checks run before anything is
 *     enqueued (the only HIP calls before them query the current device and
 *     its properties), so a rejected call has enqueued nothing.
 *   - Thread-safe and reentrant: calls may be made from several host threads
 *     and on several streams at once. The library-owned split-K workspace
 *     (gemm_f32, gemm_f32_general with a null workspace) is a small pool of
 *     device buffers per device; a call takes a buffer that no pending work
 *     can still use, or makes its stream wait (on the device, through an
 *     event) for the buffer's previous user. No entry point synchronises the
 *     device or blocks the host on GPU work.
 *   - Plans depend on the current device's compute-unit count (its
 *     multiProcessorCount; 256 on MI355X); query functions that launch
 *     nothing plan for 256 when no device can be queried.
 */
#ifndef LIBGEMM_GEMM_H
#define LIBGEMM_GEMM_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  GEMM_OK = 0,
  GEMM_ERR_INVALID_DIM = 1,      /* M, N or K negative, or a size too large to index */
  GEMM_ERR_NULL_PTR = 2,         /* null A, B or C that the call would access
                                    (A, B when M, N, K > 0; C when M, N > 0) */
  GEMM_ERR_ALIAS = 3,            /* C overlaps A or B */
  GEMM_ERR_WORKSPACE = 4,        /* workspace missing or smaller than required */
  GEMM_ERR_INVALID_PLAN = 5,     /* unknown kernel id, split count < 1 or unusable split_tail */
  GEMM_ERR_HIP = 6,              /* a HIP call failed; see gemm_last_hip_error() */
  GEMM_ERR_UNSUPPORTED_DEVICE = 7, /* the current device is not gfx950 */
  GEMM_ERR_CAPTURING = 8,         /* the stream is capturing a graph and the plan
                                     needs the library-owned workspace (pass a
                                     workspace: gemm_f32_ex, gemm_f32_with_plan,
                                     gemm_f32_general) */
  GEMM_ERR_SCRATCH_LIMIT = 9      /* gemm_f32_noalloc: the plan's partial sums need
                                     more than its static scratch buffer */
};

/* Kernel identifiers for explicit plans. Tile = the BM x BN output block one
 * workgroup computes, K step = the slice of K staged in LDS per barrier.
 * "mfma32" kernels use v_mfma_f32_32x32x2_f32, "mfma16" kernels
 * v_mfma_f32_16x16x4_f32; both are full FP32. */
enum {
  GEMM_KERNEL_AUTO = 0,            /* let the planner choose */
  GEMM_KERNEL_MFMA_256x256 = 1,    /* mfma32, 256x256 tile, K step 16, 4 waves of 128x128 */
  GEMM_KERNEL_MFMA_256x128 = 2,    /* mfma32, 256x128 tile, K step 16, 4 waves of 128x64 */
  GEMM_KERNEL_MFMA_128x128 = 3,    /* mfma32, 128x128 tile, K step 16, 4 waves of 64x64 */
  GEMM_KERNEL_MFMA_64x64 = 4,      /* mfma32, 64x64 tile, K step 16, 4 waves of 32x32 */
  GEMM_KERNEL_MFMA_256x256_W8 = 5, /* mfma32, 256x256 tile, K step 16, 8 waves of 128x64
                                      (shapes needing 4-byte loads: the 4-wave kernel) */
  GEMM_KERNEL_VALU_64x64 = 10,     /* vector FMA, 64x64 tile, K step 16, 4x4 outputs per lane */
  GEMM_KERNEL_MFMA16_256x128 = 13,    /* mfma16, 256x128 tile, K step 32, 4 waves of 128x64 */
  GEMM_KERNEL_MFMA16_128x128 = 14,    /* mfma16, 128x128 tile, K step 32, 4 waves of 64x64 */
  GEMM_KERNEL_MFMA16_64x64 = 15,      /* mfma16, 64x64 tile, K step 32, 4 waves of 32x32 */
  GEMM_KERNEL_MFMA16_128x128_K16 = 17, /* mfma16, 128x128 tile, K step 16, 4 waves of 64x64 */
  GEMM_KERNEL_MFMA16_256x128_K16 = 18, /* mfma16, 256x128 tile, K step 16, 4 waves of 128x64
                                          (K or N not a multiple of 4, or A or B not
                                          16-byte aligned: the mfma32 kernel of this tile) */
  GEMM_KERNEL_MFMA_128x128_W1 = 19,    /* mfma32, 128x128 tile, K step 16, one wave */
  GEMM_KERNEL_MFMA_64x64_W1 = 21,      /* mfma32, 64x64 tile, K step 16, one wave */
  /* Kernels fed by direct global->LDS copies through a ring of LDS stages
   * (any K and N). When a tile's copy offsets would pass 2^31 bytes, a plain
   * product runs the register-staged kernel of the same tile instead, the
   * general form runs in K passes, and a split_tail plan is rejected. */
  GEMM_KERNEL_DMA32_256x256_W8 = 30,    /* mfma32, 256x256, K step 16, 8 waves, 4 stages */
  GEMM_KERNEL_DMA32_128x128_W4 = 33,    /* mfma32, 128x128, K step 16, 4 waves, 4 stages */
  GEMM_KERNEL_DMA16_128x128_W4 = 34,    /* mfma16, 128x128, K step 16, 4 waves, 4 stages */
  GEMM_KERNEL_DMA32_256x256_W8_S3 = 35, /* mfma32, 256x256, K step 16, 8 waves, 3 stages */
  GEMM_KERNEL_DMA16_64x64 = 36,         /* mfma16, 64x64, K step 32, 4 waves, 4 stages */
  GEMM_KERNEL_DMA32_64x64 = 37,         /* mfma32, 64x64, K step 16, 4 waves, 4 stages */
  GEMM_KERNEL_DMA16_128x64 = 38,        /* mfma16, 128x64, K step 32, 4 waves, 4 stages */
  GEMM_KERNEL_DMA32_128x128_W8 = 39,    /* mfma32, 128x128, K step 16, 8 waves of 64x32, 4 stages */
  GEMM_KERNEL_DMA32_64x64_S3 = 45,      /* mfma32, 64x64, K step 16, 4 waves, 3 stages */
  GEMM_KERNEL_DMA32_128x128_W8_S3 = 46, /* mfma32, 128x128, K step 16, 8 waves of 64x32, 3 stages */
  GEMM_KERNEL_DMA16_96x96_S3 = 47,      /* mfma16, 96x96, K step 32, 4 waves of 48x48, 3 stages;
                                         * no register-staged counterpart: a plan whose copy
                                         * offsets would pass 2^31 bytes is rejected */
  /* The optimisation ladder of the yekq.top LeetGPU walkthrough (sections v0
   * to v3; its v4 is GEMM_KERNEL_VALU_64x64), for comparison only. */
  GEMM_KERNEL_LADDER_V0 = 40,  /* one output per lane, lanes along rows (uncoalesced), 16x16 */
  GEMM_KERNEL_LADDER_V1 = 41,  /* one output per lane, lanes along columns, 16x16 */
  GEMM_KERNEL_LADDER_V2 = 42,  /* 16x16 LDS tiles, two barriers per 16-wide K phase */
  GEMM_KERNEL_LADDER_V3 = 43   /* 16x64 tile, 4 outputs per lane along N, LDS K phases of 16 */
};

/* An execution plan: which kernel, and how many contiguous K ranges
 * ("split-K") the contraction is cut into. k_chunk is the length of each
 * range (a multiple of the kernel's K step); split_k = ceil(K / k_chunk).
 *
 * split_tail = 0: every output tile is split into split_k K ranges.
 * split_tail = 1 (copy-fed kernels, ids 30-39 and 45-47, only): the output tiles
 * are taken in rounds of one per CU (256 on MI355X); the tiles of the whole rounds are
 * computed over all of K and stored straight into C, and only the tiles of
 * the last, partial round are split into split_k K ranges, so that the last
 * round's work is spread over all CUs. With fewer tiles than CUs this is the
 * same as split_tail = 0; with a whole number of rounds nothing is split. */
typedef struct gemm_plan {
  int kernel;
  int split_k;
  int k_chunk;
  int split_tail;
} gemm_plan_t;

/* C = A x B with the planner's choice of kernel and split. When that plan
 * splits K, the partial sums go to a library-owned workspace: per device, up
 * to 8 buffers allocated (hipMalloc) on first need, each reused once the
 * work that last used it has completed or is ordered before this call's on
 * the same stream; calls that overlap on other streams get a buffer of their
 * own or wait for one on the device. A buffer is freed only to make room for
 * a larger one, and only once no pending work can use it. If no buffer can
 * be had the call runs the plan's kernel unsplit. Not for graph capture when
 * the plan splits K (GEMM_ERR_CAPTURING): pass a workspace (gemm_f32_ex)
 * there. Returns a status code. */
int gemm_f32(const float *A, const float *B, float *C, int M, int N, int K,
             hipStream_t stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. C = A x B
 * exactly as gemm_f32 computes it (the same plan, so the same bits), with the
 * split-K partial sums in a static device buffer of
 * gemm_f32_noalloc_scratch_bytes() bytes (64 MiB) that the library holds on
 * each device it runs on until the process ends, instead of an allocated
 * workspace. The call makes no allocation (no hipMalloc, hipFree or
 * allocating library routine) and no memset: every partial sum is written
 * before it is read, so nothing needs clearing. Limit: when the plan's
 * partial sums need more than the buffer (gemm_f32_workspace_bytes(M, N, K) >
 * gemm_f32_noalloc_scratch_bytes()) the call returns GEMM_ERR_SCRATCH_LIMIT
 * and enqueues nothing; plans that do not split K need none of it. All calls
 * on one device share that device's buffer: two such calls whose work
 * overlaps in time on one device (different streams, or a graph replayed
 * while another call runs) race and give wrong results; calls ordered on one
 * stream do not. Returns a status code. */
int gemm_f32_noalloc(const float *A, const float *B, float *C, int M, int N, int K,
                     hipStream_t stream);

/* Size in bytes of gemm_f32_noalloc's static scratch buffer. */
size_t gemm_f32_noalloc_scratch_bytes(void);

/* Bytes of workspace the planner's plan for (M, N, K) needs:
 * 4 * split_k * M * N when it splits K (one M x N slab per K range, also
 * when only the last round of tiles is split), else 0. Returns 0 for invalid
 * dims. */
size_t gemm_f32_workspace_bytes(int M, int N, int K);

/* As gemm_f32, with a caller-owned device workspace of workspace_bytes bytes
 * (at least gemm_f32_workspace_bytes(M, N, K); may be null when that is 0).
 * The workspace must not be used by other work until this call's work has
 * completed on `stream`. Returns GEMM_ERR_WORKSPACE if it is too small. */
int gemm_f32_ex(const float *A, const float *B, float *C, int M, int N, int K,
                void *workspace, size_t workspace_bytes, hipStream_t stream);

/* The planner's plan for (M, N, K) on the current device, written to *plan.
 * Returns a status code. */
int gemm_f32_plan(int M, int N, int K, gemm_plan_t *plan);

/* The planner's plan for (M, N, K) on a device of num_cus compute units
 * (num_cus >= 1; GEMM_ERR_INVALID_DIM otherwise): the rounds of tiles it
 * costs, and a split tail's whole rounds, are num_cus tiles each. For
 * planning ahead for another device, and for tests. */
int gemm_f32_plan_cus(int M, int N, int K, int num_cus, gemm_plan_t *plan);

/* Workspace bytes an explicit plan needs (0 for an invalid plan or dims). Only
 * plan->kernel, plan->split_k and plan->split_tail are read. */
size_t gemm_f32_plan_workspace_bytes(int M, int N, int K, const gemm_plan_t *plan);

/* C = A x B with an explicit plan (plan->kernel, plan->split_k,
 * plan->split_tail; split_k is clamped to the number of K steps).
 * kernel = GEMM_KERNEL_AUTO means the planner's choice. workspace as for
 * gemm_f32_ex. GEMM_ERR_INVALID_PLAN for split_tail other than 0 or 1, or 1
 * with a kernel that is not copy-fed or whose copy offsets would not fit
 * for this shape. Returns a status code. */
int gemm_f32_with_plan(const float *A, const float *B, float *C, int M, int N, int K,
                       const gemm_plan_t *plan, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* The general form, with the argument order of the BLAS SGEMM call of the
 * yekq.top LeetGPU walkthrough's cuBLAS reference section, for row-major
 * storage:
 *
 *   C <- alpha * op(A) * op(B) + beta * C,   op(A) M x K, op(B) K x N, C M x N
 *
 *   trans_a == 0: A is stored M x K, element (i, k) at A[i*lda + k], lda >= K;
 *   trans_a != 0: A is stored K x M (op(A) = A^T), element (i, k) of op(A) at
 *                 A[k*lda + i], lda >= M;
 *   trans_b == 0: B is stored K x N, element (k, j) at B[k*ldb + j], ldb >= N;
 *   trans_b != 0: B is stored N x K, element (k, j) of op(B) at B[j*ldb + k],
 *                 ldb >= K;
 *   element (i, j) of C at C[i*ldc + j], ldc >= N. Every leading dimension is
 *   at least 1. Elements between a row's end and its stride are neither read
 *   (A, B, C) nor written (C).
 *
 * BLAS conventions: beta == 0 means C is not read (NaN there does not
 * propagate); alpha == 0 or K == 0 means A and B are not read (and may be
 * null) and C <- beta * C (+0.0 when beta == 0). The sum is in FP32 as for
 * gemm_f32; then each output is fmaf(alpha, sum, fl(beta * c)): beta * c is
 * rounded to FP32 on its own and then added by one fused multiply-add (two
 * roundings in all), or fl(alpha * sum) when beta == 0. alpha = 1, beta = 0,
 * no transposes and dense strides give bit-for-bit the result of gemm_f32
 * with the same plan.
 *
 * workspace: null to use the library's split-K workspace (as gemm_f32; not
 * while the stream captures a graph when the plan splits K:
 * GEMM_ERR_CAPTURING), else a caller-owned buffer of at least
 * gemm_f32_general_workspace_bytes(...) bytes (GEMM_ERR_WORKSPACE if
 * smaller). A, B, C overlapping: C's extent (first to last element) must not
 * overlap A's or B's (GEMM_ERR_ALIAS). Operands whose rows are so long that
 * one 64-row tile spans 2^31 bytes are rejected (GEMM_ERR_INVALID_DIM);
 * an operand whose K range would span 2^31 bytes is processed in several
 * K passes, each after the first accumulating into C. Returns a status.
 *
 * Column-major data (the BLAS convention): a column-major r x c matrix with
 * leading dimension ld is the row-major c x r matrix with row stride ld, its
 * transpose, and (op(A) op(B))^T = op(B)^T op(A)^T. So the column-major
 * product C = alpha * op(A) op(B) + beta * C (A, B, C column-major with
 * leading dimensions lda, ldb, ldc) is
 *   gemm_f32_general(trans_b, trans_a, N, M, K, alpha, B, ldb, A, lda, beta,
 *                    C, ldc, ...). */
int gemm_f32_general(int trans_a, int trans_b, int M, int N, int K, float alpha, const float *A,
                     int lda, const float *B, int ldb, float beta, float *C, int ldc,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes gemm_f32_general needs for these shapes and strides
 * (0 when it needs none, or for invalid arguments). */
size_t gemm_f32_general_workspace_bytes(int trans_a, int trans_b, int M, int N, int K, int lda,
                                        int ldb);

/* Static, human-readable name of a kernel id ("unknown" otherwise). */
const char *gemm_kernel_name(int kernel);

/* Static, human-readable text of a status code. */
const char *gemm_status_string(int status);

/* The hipError_t of the last failed HIP call made by this library on the
 * calling thread (0 if none). */
int gemm_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBGEMM_GEMM_H */

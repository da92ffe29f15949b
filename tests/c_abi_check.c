/* A C99 caller of libgemm: include/gemm.h compiled as C, the library linked
 * directly (no Python). Exercises the host-side contract that needs no GPU:
 * plans, workspace sizes, argument checks (all made before any HIP call) and
 * the static strings. Prints one line per check for the test to compare. */
#include <stdint.h>
#include <stdio.h>

#include "gemm.h"

static const float *fake(uintptr_t a) { return (const float *)a; }

int main(void) {
  const int shapes[][3] = {{128, 112, 96}, {1024, 1024, 512}, {1001, 777, 513},
                           {4096, 4096, 4096}, {512, 512, 131072}, {1536, 1536, 1536}};
  for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i) {
    const int M = shapes[i][0], N = shapes[i][1], K = shapes[i][2];
    gemm_plan_t p;
    const int st = gemm_f32_plan(M, N, K, &p);
    printf("plan %d %d %d %d %s %d %d %d %zu %zu\n", M, N, K, st, gemm_kernel_name(p.kernel),
           p.split_k, p.k_chunk, p.split_tail, gemm_f32_workspace_bytes(M, N, K),
           gemm_f32_plan_workspace_bytes(M, N, K, &p));
  }
  const float *A = fake(0x7f0000000000u), *B = fake(0x7f1000000000u);
  float *C = (float *)(uintptr_t)0x7f2000000000u;
  printf("negative %d\n", gemm_f32(A, B, C, -1, 4, 4, 0));
  printf("null %d\n", gemm_f32(NULL, B, C, 4, 4, 4, 0));
  printf("alias %d\n", gemm_f32(A, B, (float *)(uintptr_t)0x7f0000000010u, 4, 4, 4, 0));
  printf("workspace %d\n", gemm_f32_ex(A, B, C, 512, 512, 131072, NULL, 0, 0));
  gemm_plan_t bad = {99, 1, 0, 0};
  printf("plan_kernel %d\n", gemm_f32_with_plan(A, B, C, 8, 8, 8, &bad, NULL, 0, 0));
  gemm_plan_t bad_tail = {GEMM_KERNEL_MFMA_64x64, 2, 0, 1};
  printf("plan_tail %d\n", gemm_f32_with_plan(A, B, C, 8, 8, 8, &bad_tail, NULL, 0, 0));
  printf("general_ld %d\n",
         gemm_f32_general(0, 0, 4, 4, 4, 1.0f, A, 3, B, 4, 0.0f, C, 4, NULL, 0, 0));
  printf("general_ws %zu\n", gemm_f32_general_workspace_bytes(1, 1, 256, 256, 8192, 256, 8192));
  for (int s = 0; s <= 8; ++s) printf("status %d %s\n", s, gemm_status_string(s));
  printf("kernel_auto %s\n", gemm_kernel_name(GEMM_KERNEL_AUTO));
  printf("last_hip_error %d\n", gemm_last_hip_error());
  return 0;
}

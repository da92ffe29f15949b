"""gemm_f32_noalloc: the no-allocation variant of gemm_f32 (split-K partial
sums in a static device buffer instead of an allocated workspace), through
the C ABI, checked against gemm_f32 on the same inputs: the same plan, so
the same bits. Two calls in a row, the second on a smaller input, so the
second reuses the buffer the first left behind; integer inputs bit-exact
against the exact product; a plan whose partial sums exceed the buffer is
refused before anything is enqueued."""
import numpy as np
import pytest

import gemm_inputs
import oracle
from fp32_gemm_07_amd import binding
from gpu_util import nan_buffer, say, to_dev, torch
from parity import assert_bits_equal, assert_within_bound

pytestmark = pytest.mark.gpu


def _both(A, B):
    """(gemm_f32_noalloc result, gemm_f32 result) for A x B, C NaN-filled."""
    t = torch()
    M, K = A.shape
    N = B.shape[1]
    dA, dB = to_dev(A), to_dev(B)
    c1, c2 = nan_buffer(M * N), nan_buffer(M * N)
    h = t.cuda.current_stream().cuda_stream
    binding.gemm_f32_noalloc(dA, dB, c1, M, N, K, h)
    binding.gemm_f32(dA, dB, c2, M, N, K, h)
    t.cuda.synchronize()
    return c1.cpu().numpy().reshape(M, N), c2.cpu().numpy().reshape(M, N)


# (M, K, N): the long-K workload (K split 16 ways: 16 MiB of partial sums),
# then smaller split plans, a split-tail plan and an unsplit one.
CALLS = [(512, 131072, 512), (256, 16384, 256), (1792, 1792, 1792), (100, 3000, 70),
         (1001, 513, 777)]


def test_noalloc_matches_gemm_f32_call_after_call():
    scratch = binding.gemm_f32_noalloc_scratch_bytes()
    assert scratch == 64 << 20
    for i, (M, K, N) in enumerate(CALLS):
        need = binding.gemm_f32_workspace_bytes(M, N, K)
        assert need <= scratch
        say(f"noalloc call {i}: {M}x{K}x{N} plan {binding.gemm_f32_plan(M, N, K)} "
            f"partial sums {need} B")
        A, B = gemm_inputs.draw(M, K, N, "uniform", seed=200 + i)
        got, want = _both(A, B)
        assert_bits_equal(got, want, f"noalloc vs gemm_f32 {M}x{K}x{N}")
        if M * N * K <= (1 << 31):
            C_ref, S = oracle.gemm(A, B)
            assert_within_bound(got, C_ref, S, f"noalloc {M}x{K}x{N}")
    M, K, N = CALLS[0]
    assert binding.gemm_f32_plan(M, N, K).split_k > 1


def test_noalloc_integers_bit_exact_second_call_smaller():
    for i, (M, K, N) in enumerate([(512, 65536, 512), (128, 8192, 128)]):
        say(f"noalloc integers {M}x{K}x{N}")
        A, B = gemm_inputs.draw(M, K, N, "int", seed=300 + i)
        got, want = _both(A, B)
        C_ref = oracle.gemm_i64(A.astype(np.int64), B.astype(np.int64)).astype(np.float32)
        assert_bits_equal(got, C_ref, f"noalloc int {M}x{K}x{N}")
        assert_bits_equal(want, C_ref, f"gemm_f32 int {M}x{K}x{N}")


def test_noalloc_refuses_plans_beyond_its_buffer():
    """1280 x 65536 x 1280 splits K 16 ways (the last round of tiles only):
    its partial sums need 100 MiB, more than the buffer, so the call is
    refused with GEMM_ERR_SCRATCH_LIMIT and C is left untouched; the same
    product through gemm_f32 runs."""
    t = torch()
    M, K, N = 1280, 65536, 1280
    need = binding.gemm_f32_workspace_bytes(M, N, K)
    say(f"noalloc over the limit {M}x{K}x{N}, partial sums {need} B")
    assert need > binding.gemm_f32_noalloc_scratch_bytes()
    dA = t.zeros((M, K), dtype=t.float32, device="cuda:0")
    dB = t.zeros((K, N), dtype=t.float32, device="cuda:0")
    dC = nan_buffer(M * N)
    with pytest.raises(binding.GemmError) as e:
        binding.gemm_f32_noalloc(dA, dB, dC, M, N, K, t.cuda.current_stream().cuda_stream)
    assert e.value.status == binding.GEMM_ERR_SCRATCH_LIMIT
    t.cuda.synchronize()
    assert t.isnan(dC).all()
    binding.gemm_f32(dA, dB, dC, M, N, K, t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    assert (dC == 0).all()

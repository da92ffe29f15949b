"""The blocked, zero-padded, split-K mechanism reproduces the oracle (CPU only)."""
import numpy as np
import pytest

import gemm_inputs
import oracle
from parity import assert_bits_equal, assert_within_bound
from tile_model import tiled_gemm


def test_lesson10_simulation_case():
    """The lesson's own check: 35x45 @ 45x25 randn (seed 42), tile 16, agrees
    with the reference to the lesson's allclose tolerance (atol 1e-5, NumPy's
    default rtol 1e-5); here the reference is the oracle."""
    A, B = gemm_inputs.draw_lesson10_case()
    C_ref, S = oracle.gemm(A, B)
    C = tiled_gemm(A, B, 16, 16, 16)
    assert np.allclose(C, C_ref, atol=1e-5)
    assert_within_bound(C, C_ref, S, "lesson10 tile model")


@pytest.mark.parametrize("M,K,N,BM,BN,BK,splits", [
    (35, 45, 25, 16, 16, 16, 1),
    (70, 97, 33, 32, 32, 8, 1),
    (128, 96, 112, 64, 64, 16, 1),
    (65, 130, 47, 32, 64, 16, 3),
    (33, 513, 17, 32, 32, 16, 4),
])
def test_tile_model_matches_oracle(M, K, N, BM, BN, BK, splits):
    A, B = gemm_inputs.draw(M, K, N, "uniform", seed=M + K + N)
    C_ref, S = oracle.gemm(A, B)
    assert_within_bound(tiled_gemm(A, B, BM, BN, BK, splits), C_ref, S, "tile model")


@pytest.mark.parametrize("M,K,N,BM,BN,BK,splits", [
    (35, 45, 25, 16, 16, 16, 1),
    (65, 130, 47, 32, 64, 16, 3),
    (33, 513, 17, 32, 32, 16, 5),
])
def test_tile_model_bit_exact_on_integers(M, K, N, BM, BN, BK, splits):
    A, B = gemm_inputs.draw(M, K, N, "int", seed=3)
    C_ref, _ = oracle.gemm(A, B)
    assert_bits_equal(tiled_gemm(A, B, BM, BN, BK, splits), C_ref, "tile model int")


def test_garbage_instead_of_zero_fill_is_detected():
    """Without zero fill the padded lanes add junk: the bound catches it."""
    A, B = gemm_inputs.draw(35, 45, 25, "uniform", seed=1)
    C_ref, S = oracle.gemm(A, B)
    Apad = np.concatenate([A, np.ones((35, 3), np.float32)], axis=1)  # K tail reads 3 junk columns
    Bpad = np.concatenate([B, np.ones((3, 25), np.float32)], axis=0)
    with pytest.raises(AssertionError):
        assert_within_bound(tiled_gemm(Apad, Bpad, 16, 16, 16), C_ref, S, "junk")

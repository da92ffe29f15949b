"""The blocked, zero-padded, split-K mechanism reproduces the oracle (CPU only)."""
import numpy as np
import pytest

import gemm_inputs
import oracle
from parity import assert_bits_equal, assert_within_bound
from tile_model import tile_order, tiled_gemm


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


@pytest.mark.parametrize("M,K,N,BM,BN,tail_round,splits", [
    (50, 97, 40, 16, 16, 4, 3),      # 4 x 3 tiles = 3 whole rounds of 4: nothing split
    (60, 97, 45, 16, 16, 5, 3),      # 4 x 3 = 12 tiles: two rounds of 5 whole, 2 split
    (70, 130, 47, 16, 16, 8, 4),     # 5 x 3 = 15 tiles: one round of 8 whole, 7 split
    (33, 513, 17, 16, 16, 4, 2),     # 3 x 2 = 6 tiles: 4 whole, 2 split
])
def test_split_tail_model(M, K, N, BM, BN, tail_round, splits):
    """Split tail on the CPU model: within the bound of the oracle, bitwise on
    integers, and every tile equal to the unsplit model's (whole rounds) or to
    the split-every-tile model's (last round) bit for bit."""
    for dist in ("uniform", "int"):
        A, B = gemm_inputs.draw(M, K, N, dist, seed=M + N)
        C_ref, S = oracle.gemm(A, B)
        C = tiled_gemm(A, B, BM, BN, 16, splits, tail_round=tail_round)
        if dist == "int":
            assert_bits_equal(C, C_ref, "split tail model int")
            continue
        assert_within_bound(C, C_ref, S, "split tail model")
        one = tiled_gemm(A, B, BM, BN, 16, 1)
        every = tiled_gemm(A, B, BM, BN, 16, splits)
        order = tile_order(-(-M // BM), -(-N // BN))
        whole = len(order) // tail_round * tail_round
        for i, (r, c) in enumerate(order):
            rs, cs = slice(r * BM, (r + 1) * BM), slice(c * BN, (c + 1) * BN)
            want = one if i < whole else every
            assert_bits_equal(C[rs, cs], want[rs, cs], f"tile {i}")


def test_garbage_instead_of_zero_fill_is_detected():
    """Without zero fill the padded lanes add junk: the bound catches it."""
    A, B = gemm_inputs.draw(35, 45, 25, "uniform", seed=1)
    C_ref, S = oracle.gemm(A, B)
    Apad = np.concatenate([A, np.ones((35, 3), np.float32)], axis=1)  # K tail reads 3 junk columns
    Bpad = np.concatenate([B, np.ones((3, 25), np.float32)], axis=0)
    with pytest.raises(AssertionError):
        assert_within_bound(tiled_gemm(Apad, Bpad, 16, 16, 16), C_ref, S, "junk")

"""The seeded input generators (CPU only)."""
import numpy as np
import pytest

import gemm_inputs


def test_deterministic_and_distinct_per_seed():
    A1, B1 = gemm_inputs.draw(33, 17, 9, "uniform", 5)
    A2, B2 = gemm_inputs.draw(33, 17, 9, "uniform", 5)
    A3, _ = gemm_inputs.draw(33, 17, 9, "uniform", 6)
    assert A1.tobytes() == A2.tobytes() and B1.tobytes() == B2.tobytes()
    assert A1.tobytes() != A3.tobytes()
    assert A1.dtype == np.float32 and A1.flags.c_contiguous and A1.shape == (33, 17)
    assert B1.shape == (17, 9)


def test_uniform_range_is_half_open_minus_one_to_one():
    A, B = gemm_inputs.draw(512, 512, 512, "uniform", 0)
    for X in (A, B):
        assert X.min() >= -1.0 and X.max() < 1.0
        assert abs(float(X.mean())) < 0.01
        # values are multiples of 2^-23: exact in float32
        assert np.all((X.astype(np.float64) * 2 ** 23) % 1 == 0)


def test_normal_scaled_by_inverse_sqrt_k():
    A, B = gemm_inputs.draw(256, 4096, 64, "normal", 3)
    assert float(A.std()) == pytest.approx(1 / 64, rel=0.02)
    assert float(B.std()) == pytest.approx(1 / 64, rel=0.02)


@pytest.mark.parametrize("K,r", [(96, 16), (4096, 16), (65536, 16), (131072, 11), (1 << 24, 1)])
def test_integer_range_keeps_sums_exact(K, r):
    assert gemm_inputs.int_range(K) == r
    assert K * r * r <= 2 ** 24


def test_integer_inputs_are_integers_in_range():
    A, B = gemm_inputs.draw(64, 131072 // 64, 32, "int", 1)
    r = gemm_inputs.int_range(131072 // 64)
    assert np.all(A == np.round(A)) and np.abs(A).max() <= r


def test_standing_workloads():
    names = [w.name for w in gemm_inputs.WORKLOADS]
    assert len(names) == 5 and len(set(names)) == 5
    w = gemm_inputs.BY_NAME["irregular_1001x513x777"]
    assert (w.M, w.K, w.N, w.seed) == (1001, 513, 777, 2)
    w4 = gemm_inputs.BY_NAME["square_4096"]
    assert w4.dist == "normal" and w4.seed == 3


def test_sample_indices_cover_corners_and_stay_in_range():
    r, c = gemm_inputs.sample_indices(1001, 777, 100)
    assert r.min() >= 0 and r.max() < 1001 and c.min() >= 0 and c.max() < 777
    pts = set(zip(r.tolist(), c.tolist()))
    assert {(0, 0), (0, 776), (1000, 0), (1000, 776)} <= pts

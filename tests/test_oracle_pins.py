"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test ties the oracle to something the pages or the mathematics fix:
hand-worked products of the element-wise definition (golden file), the
identity, all-ones inputs (C = K), an exact integer product checked against
pure-Python integer loops, exact rational arithmetic (error bound), a
library routine on the same definition (NumPy matmul in float64), the
transpose identity (AB)^T = B^T A^T, and additivity over K. A plausible slip
in the oracle (a dropped term, a sign, a stride, a transposed operand, an
FP32 accumulator, a missing absolute value, a wrong sampled index) fails at
least one of them.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import gemm_inputs
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_hand_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "hand_products.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            if key == "case":
                cur = {"name": vals[0], "M": int(vals[1]), "K": int(vals[2]), "N": int(vals[3])}
                cases.append(cur)
            else:
                cur[key] = [float(v) for v in vals]
    return cases


HAND = _read_hand_cases()


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


@pytest.mark.parametrize("case", HAND, ids=[c["name"] for c in HAND])
def test_hand_worked_products(case):
    M, K, N = case["M"], case["K"], case["N"]
    A = np.array(case["A"], dtype=np.float32).reshape(M, K)
    B = np.array(case["B"], dtype=np.float32).reshape(K, N)
    want = np.array(case["C"], dtype=np.float32).reshape(M, N)
    C, S = oracle.gemm(A, B)
    assert C.dtype == np.float32 and C.shape == (M, N)
    np.testing.assert_array_equal(C.view(np.uint32), want.view(np.uint32))
    if "S" in case:
        np.testing.assert_array_equal(S, np.array(case["S"]).reshape(M, N))
    # the entry-wise routine agrees with the full one on the same definition
    rr, cc = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    vals, svals = oracle.gemm_entries(A, B, rr.ravel(), cc.ravel())
    np.testing.assert_array_equal(vals.view(np.uint32), want.ravel().view(np.uint32))
    np.testing.assert_array_equal(svals, S.ravel())


def _python_int_gemm(A, B, M, K, N):
    return [[sum(A[i][k] * B[k][j] for k in range(K)) for j in range(N)] for i in range(M)]


@pytest.mark.parametrize("M,K,N,seed", [(1, 1, 1, 0), (3, 5, 2, 1), (7, 4, 9, 2), (5, 33, 6, 3),
                                        (2, 0, 3, 4)])
def test_integer_oracle_matches_python_loops(M, K, N, seed):
    rng = np.random.default_rng(seed)
    A = rng.integers(-16, 17, size=(M, K))
    B = rng.integers(-16, 17, size=(K, N))
    want = _python_int_gemm(A.tolist(), B.tolist(), M, K, N)
    got = oracle.gemm_i64(A, B)
    assert got.tolist() == want


@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (4, 7, 3), (33, 65, 31), (128, 96, 112)])
def test_identity(M, K, N):
    A, B = gemm_inputs.draw(M, K, N, "uniform", seed=11)
    I_K = np.eye(K, dtype=np.float32)
    I_M = np.eye(M, dtype=np.float32)
    C1, _ = oracle.gemm(A, I_K)
    C2, _ = oracle.gemm(I_K, B)
    C3, _ = oracle.gemm(I_M, A)
    np.testing.assert_array_equal(C1.view(np.uint32), A.view(np.uint32))
    np.testing.assert_array_equal(C2.view(np.uint32), B.view(np.uint32))
    np.testing.assert_array_equal(C3.view(np.uint32), A.view(np.uint32))


@pytest.mark.parametrize("M,K,N", [(3, 1, 5), (4, 7, 2), (2, 96, 3), (5, 513, 4), (3, 131072, 5)])
def test_all_ones_gives_K(M, K, N):
    A = np.ones((M, K), np.float32)
    B = np.ones((K, N), np.float32)
    C, S = oracle.gemm(A, B)
    assert np.all(C == np.float32(K))
    assert np.all(S == float(K))


def test_empty_sum_is_positive_zero():
    A = np.zeros((3, 0), np.float32)
    B = np.zeros((0, 4), np.float32)
    C, S = oracle.gemm(A, B)
    assert C.shape == (3, 4)
    assert np.all(C.view(np.uint32) == 0)  # +0.0 bits
    assert np.all(S == 0)
    # all products -0.0: the sum starting at +0.0 stays +0.0
    C2, _ = oracle.gemm(np.full((2, 3), -0.0, np.float32), np.ones((3, 2), np.float32))
    assert np.all(C2.view(np.uint32) == 0)


def test_degenerate_shapes():
    C, S = oracle.gemm(np.zeros((0, 5), np.float32), np.zeros((5, 3), np.float32))
    assert C.shape == (0, 3)
    C, S = oracle.gemm(np.zeros((4, 5), np.float32), np.zeros((5, 0), np.float32))
    assert C.shape == (4, 0)


@pytest.mark.parametrize("M,K,N,seed", [(8, 50, 6, 0), (5, 200, 4, 1), (3, 1000, 3, 2)])
def test_within_recursive_summation_bound_of_exact(M, K, N, seed):
    """|C_ref - exact| <= ulp(C_ref)/2 + K * 2^-53 * S (FP64 recursive summation
    error bound, then one rounding to FP32), checked in exact rationals."""
    A, B = gemm_inputs.draw(M, K, N, "uniform", seed=seed)
    C, S = oracle.gemm(A, B)
    Af = [[Fraction(float(x)) for x in row] for row in A]
    Bf = [[Fraction(float(x)) for x in row] for row in B]
    for i in range(M):
        for j in range(N):
            exact = sum(Af[i][k] * Bf[k][j] for k in range(K))
            sabs = sum(abs(Af[i][k] * Bf[k][j]) for k in range(K))
            ulp = Fraction(float(np.spacing(np.float32(abs(C[i, j])))))
            bound = ulp / 2 + K * Fraction(1, 2 ** 53) * sabs
            assert abs(Fraction(float(C[i, j])) - exact) <= bound
            assert abs(Fraction(float(S[i, j])) - sabs) <= K * Fraction(1, 2 ** 53) * sabs


@pytest.mark.parametrize("M,K,N,seed", [(64, 96, 48, 0), (33, 513, 17, 1), (128, 96, 112, 2)])
def test_agrees_with_float64_library_matmul(M, K, N, seed):
    """NumPy's float64 matmul is the same definition with another summation
    order; after one rounding to FP32 both agree to within one FP32 ulp."""
    A, B = gemm_inputs.draw(M, K, N, "uniform", seed=seed)
    C, S = oracle.gemm(A, B)
    ref = (A.astype(np.float64) @ B.astype(np.float64)).astype(np.float32)
    ulp = np.spacing(np.maximum(np.abs(C), np.abs(ref)))
    assert np.all(np.abs(C.astype(np.float64) - ref) <= ulp)
    np.testing.assert_allclose(S, np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64),
                               rtol=1e-12)


@pytest.mark.parametrize("M,K,N,seed", [(37, 45, 29, 0), (128, 96, 112, 1)])
def test_transpose_identity(M, K, N, seed):
    """(AB)^T = B^T A^T: the same products summed in the same k order."""
    A, B = gemm_inputs.draw(M, K, N, "uniform", seed=seed)
    C, S = oracle.gemm(A, B)
    Ct, St = oracle.gemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    np.testing.assert_array_equal(Ct.T.view(np.uint32), C.view(np.uint32))
    np.testing.assert_array_equal(St.T, S)


@pytest.mark.parametrize("k1", [1, 17, 48, 95])
def test_additive_over_k_on_integers(k1):
    M, K, N = 20, 96, 24
    A, B = gemm_inputs.draw(M, K, N, "int", seed=5)
    C, _ = oracle.gemm(A, B)
    C1, _ = oracle.gemm(A[:, :k1], B[:k1])
    C2, _ = oracle.gemm(A[:, k1:], B[k1:])
    np.testing.assert_array_equal(C1 + C2, C)


# Every standing shape, reduced where the full product is too large for the
# CPU suite: the reduced cases keep the full K (the accumulation length).
_INT_SHAPES = [(128, 96, 112), (1024, 512, 64), (1001, 513, 777), (64, 4096, 64), (8, 131072, 8)]


@pytest.mark.parametrize("M,K,N", _INT_SHAPES)
def test_small_integers_exact(M, K, N):
    A, B = gemm_inputs.draw(M, K, N, "int", seed=7)
    r = gemm_inputs.int_range(K)
    assert np.abs(A).max() <= r and np.abs(B).max() <= r and K * r * r <= 2 ** 24
    C, _ = oracle.gemm(A, B)
    Ci = oracle.gemm_i64(A.astype(np.int64), B.astype(np.int64))
    assert np.abs(Ci).max() <= 2 ** 24
    np.testing.assert_array_equal(C.view(np.uint32), Ci.astype(np.float32).view(np.uint32))


def test_entries_match_full_product():
    A, B = gemm_inputs.draw(70, 130, 90, "uniform", seed=3)
    C, S = oracle.gemm(A, B)
    rows, cols = gemm_inputs.sample_indices(70, 90, 500, seed=1)
    vals, svals = oracle.gemm_entries(A, B, rows, cols)
    np.testing.assert_array_equal(vals.view(np.uint32), C[rows, cols].view(np.uint32))
    np.testing.assert_array_equal(svals, S[rows, cols])


def test_result_independent_of_thread_count():
    A, B = gemm_inputs.draw(61, 77, 45, "uniform", seed=9)
    C1, S1 = oracle.gemm(A, B, threads=1)
    C3, S3 = oracle.gemm(A, B, threads=3)
    np.testing.assert_array_equal(C1.view(np.uint32), C3.view(np.uint32))
    np.testing.assert_array_equal(S1, S3)


def test_bad_arguments_raise():
    with pytest.raises(ValueError):
        oracle.gemm(np.zeros((2, 3), np.float32), np.zeros((4, 2), np.float32))
    with pytest.raises(RuntimeError):
        oracle.gemm_entries(np.zeros((2, 3), np.float32), np.zeros((3, 2), np.float32), [2], [0])


def test_special_values_follow_ieee_products_and_sums():
    """Each output is the sum over k of A[i, k] * B[k, j] and nothing else, in
    IEEE arithmetic: a NaN in A[i0, :] makes row i0 NaN; +Inf at B[k1, j1]
    gives sign(A[i, k1]) * Inf down column j1 and NaN where A[i, k1] = 0
    (0 * Inf); -Inf at B[k2, j2] with a +Inf from the same row of A's k1 makes
    NaN (Inf - Inf); every other entry is finite. Checked against Python's own
    float arithmetic entry by entry on a tiny case."""
    M, K, N = 6, 5, 4
    A, B = gemm_inputs.draw(M, K, N, "uniform", seed=9)
    A = A.astype(np.float64)
    B = B.astype(np.float64)
    A[1, 2] = np.nan
    B[3, 1] = np.inf
    A[4, 3] = 0.0
    B[0, 2] = -np.inf
    B[3, 2] = np.inf      # column 2 gets +Inf * A[i, 3] and -Inf * A[i, 0]
    A32, B32 = A.astype(np.float32), B.astype(np.float32)
    C, _ = oracle.gemm(A32, B32)
    for i in range(M):
        for j in range(N):
            want = 0.0
            for k in range(K):
                want += float(A32[i, k]) * float(B32[k, j])
            if np.isnan(want):
                assert np.isnan(C[i, j]), (i, j)
            else:
                assert C[i, j] == pytest.approx(want, rel=1e-12, abs=1e-12), (i, j)
    assert np.isnan(C[1]).all()
    assert np.isnan(C[4, 1]) and np.isinf(C[0, 1])

"""Pins of the oracle's general form, C <- alpha op(A) op(B) + beta C with
leading dimensions (CPU only).

The pages fix alpha = 1, beta = 0 and dense operands; the general form
follows the BLAS conventions of the interface the LeetGPU walkthrough's
cuBLAS reference section calls. Pinned by: hand-worked cases with padding
and unread operands filled with NaN (tests/golden/general_products.txt);
agreement with the plain oracle after explicit transposition and
re-striding; exact integer identities for alpha and beta; the S scale.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "general_products.txt")


def _load_cases():
    cases, cur = [], None
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tok = line.split()
            if tok[0] == "case":
                cur = {"name": tok[1], "ta": int(tok[2]), "tb": int(tok[3]), "M": int(tok[4]),
                       "K": int(tok[5]), "N": int(tok[6]), "alpha": float(tok[7]),
                       "beta": float(tok[8]), "lda": int(tok[9]), "ldb": int(tok[10]),
                       "ldc": int(tok[11])}
                cases.append(cur)
            else:
                cur[tok[0]] = np.array([float(x) for x in tok[1:]], np.float32)
    return cases


GENERAL = _load_cases()


def run_case(lib, c):
    return lib.gemm_general(c["ta"], c["tb"], c["M"], c["N"], c["K"], c["alpha"], c["A"], c["lda"],
                            c["B"], c["ldb"], c["beta"], c["Cin"], c["ldc"])


def case_matches(out, want):
    nan_w = np.isnan(want)
    return bool(np.array_equal(np.isnan(out), nan_w) and
                np.array_equal(out[~nan_w].view(np.uint32), want[~nan_w].view(np.uint32)))


@pytest.mark.parametrize("case", GENERAL, ids=[c["name"] for c in GENERAL])
def test_hand_worked_general_cases(case):
    out, S = run_case(oracle, case)
    assert case_matches(out, case["Cout"]), (case["name"], out, case["Cout"])
    assert np.isfinite(S).all()


def _store(X, trans, ld, rng):
    """Storage of op(X) = X: X itself (trans 0) or X^T (trans 1), rows padded
    to ld with random junk."""
    Y = X.T if trans else X
    buf = rng.standard_normal((Y.shape[0], ld)).astype(np.float32) * 1e30
    buf[:, :Y.shape[1]] = Y
    return buf.ravel()


@pytest.mark.parametrize("ta", [0, 1])
@pytest.mark.parametrize("tb", [0, 1])
@pytest.mark.parametrize("M,K,N", [(5, 7, 3), (17, 33, 9)])
def test_matches_plain_oracle_after_explicit_transposition(ta, tb, M, K, N):
    rng = np.random.default_rng(M * 100 + K + ta * 7 + tb * 13)
    X = (rng.random((M, K), dtype=np.float32) * 2 - 1)
    Y = (rng.random((K, N), dtype=np.float32) * 2 - 1)
    lda = (M if ta else K) + 3
    ldb = (K if tb else N) + 5
    ldc = N + 2
    A, B = _store(X, ta, lda, rng), _store(Y, tb, ldb, rng)
    Cin = np.full(M * ldc, np.nan, np.float32)
    out, S = oracle.gemm_general(ta, tb, M, N, K, 1.0, A, lda, B, ldb, 0.0, Cin, ldc)
    ref, S_ref = oracle.gemm(X, Y)
    got = out.reshape(M, ldc)
    assert np.array_equal(got[:, :N].view(np.uint32), ref.view(np.uint32))
    assert np.isnan(got[:, N:]).all()
    assert np.array_equal(S, S_ref)


@pytest.mark.parametrize("alpha,beta", [(3.0, -2.0), (-1.0, 1.0), (0.5, 4.0)])
def test_alpha_beta_exact_on_integers(alpha, beta):
    """Small integers (and alpha, beta with short binary expansions): every
    quantity is exact, so the result equals alpha*P + beta*C0 computed in
    Python integers/fractions."""
    rng = np.random.default_rng(11)
    M, K, N = 6, 9, 5
    X = rng.integers(-8, 9, (M, K))
    Y = rng.integers(-8, 9, (K, N))
    C0 = rng.integers(-50, 51, (M, N))
    P = [[sum(int(X[i, k]) * int(Y[k, j]) for k in range(K)) for j in range(N)] for i in range(M)]
    want = np.array([[alpha * P[i][j] + beta * int(C0[i, j]) for j in range(N)] for i in range(M)],
                    np.float32)
    out, S = oracle.gemm_general(0, 0, M, N, K, alpha, X.astype(np.float32).ravel(), K,
                                 Y.astype(np.float32).ravel(), N, beta,
                                 C0.astype(np.float32).ravel(), N)
    assert np.array_equal(out.reshape(M, N), want)
    absP = np.abs(X) @ np.abs(Y)
    assert np.array_equal(S, abs(alpha) * absP + np.abs(beta * C0))


def test_bad_arguments_rejected():
    A = np.zeros(4, np.float32)
    with pytest.raises(RuntimeError):   # lda < K
        oracle.gemm_general(0, 0, 2, 2, 2, 1.0, A, 1, A, 2, 0.0, A.copy(), 2)
    with pytest.raises(RuntimeError):   # transposed A needs lda >= M
        oracle.gemm_general(1, 0, 3, 1, 1, 1.0, A, 2, A, 1, 0.0, A.copy(), 1)
    with pytest.raises(RuntimeError):   # ldc < N
        oracle.gemm_general(0, 0, 1, 2, 1, 1.0, A, 1, A, 2, 0.0, A.copy(), 1)

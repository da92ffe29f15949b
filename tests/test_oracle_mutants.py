"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is a copy of gemm_oracle.c with one plausible slip planted in its
source, compiled with gcc into a temporary library. The same kinds of checks
that pin the real oracle (hand-worked products, all-ones inputs, the empty
sum, the exact integer product against Python loops, sampled entries against
hand values) are run on every mutant, and each mutant must fail at least one.
The real oracle must pass all of them.
"""
import os

import numpy as np
import pytest

import oracle
from test_oracle_general_pins import GENERAL, case_matches, run_case
from test_oracle_pins import HAND, _python_int_gemm

SRC = os.path.join(os.path.dirname(oracle.__file__), "gemm_oracle.c")

# (name, exact substring of gemm_oracle.c, replacement)
MUTANTS = [
    ("dropped_last_term",
     "for (int64_t k = 0; k < K; ++k) {\n          const double a = (double)A[i * K + k];",
     "for (int64_t k = 0; k < K - 1; ++k) {\n          const double a = (double)A[i * K + k];"),
    ("wrong_sign", "acc[j] += p;", "acc[j] -= p;"),
    ("b_row_stride_K", "const float *brow = B + k * N;", "const float *brow = B + k * K;"),
    ("a_transposed", "const double a = (double)A[i * K + k];", "const double a = (double)A[k * M + i];"),
    ("b_transposed", "const double p = a * (double)brow[j];", "const double p = a * (double)B[j * K + k];"),
    ("fp32_accumulator", "double *acc = (double *)malloc(sizeof(double) * (size_t)N);",
     "float *acc = (float *)malloc(sizeof(float) * (size_t)N);"),
    ("abs_dropped", "sab[j] += fabs(p);", "sab[j] += p;"),
    ("c_stored_transposed", "C[i * N + j] = (float)acc[j];", "C[j * M + i] = (float)acc[j];"),
    ("negative_zero_start", "acc[j] = 0.0;", "acc[j] = -0.0;"),
    ("entries_wrong_column", "(double)A[i * K + k] * (double)B[k * N + j];",
     "(double)A[i * K + k] * (double)B[k * N + i];"),
    ("i64_adds_instead_of_multiplies", "crow[j] += a * brow[j];", "crow[j] += a + brow[j];"),
    # the general form
    ("general_lda_taken_as_K", "(double)A[i * lda + k];", "(double)A[i * K + k];"),
    ("general_transposed_a_indexed_as_plain", "(double)A[k * lda + i]", "(double)A[i * lda + k]"),
    ("general_transposed_b_indexed_as_plain", "(double)B[j * ldb + k]", "(double)B[k * ldb + j]"),
    ("general_ldc_taken_as_N", "C[i * ldc + j] = (float)r;", "C[i * N + j] = (float)r;"),
    ("general_alpha_not_applied", "r = (double)alpha * sum + (double)beta * c;",
     "r = sum + (double)beta * c;"),
    ("general_beta_not_applied", "r = (double)alpha * sum + (double)beta * c;",
     "r = (double)alpha * sum + c;"),
    ("general_c_read_when_beta_zero", "const double c = beta != 0.0f ? (double)C[i * ldc + j] : 0.0;",
     "const double c = (double)C[i * ldc + j];"),
    ("general_ab_read_when_alpha_zero", "const int use_ab = alpha != 0.0f && K > 0;",
     "const int use_ab = K > 0;"),
]


def _pin_failures(lib: "oracle.OracleLib"):
    """Run the pin checks against one compiled oracle; return the names that fail."""
    failed = []

    for case in HAND:
        M, K, N = case["M"], case["K"], case["N"]
        A = np.array(case["A"], np.float32).reshape(M, K)
        B = np.array(case["B"], np.float32).reshape(K, N)
        want = np.array(case["C"], np.float32).reshape(M, N)
        C, S = lib.gemm(A, B)
        if not np.array_equal(C.view(np.uint32), want.view(np.uint32)):
            failed.append("hand:" + case["name"])
        if "S" in case and not np.array_equal(S, np.array(case["S"]).reshape(M, N)):
            failed.append("hand_S:" + case["name"])
        rr, cc = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        vals, _ = lib.gemm_entries(A, B, rr.ravel(), cc.ravel())
        if not np.array_equal(vals.view(np.uint32), want.ravel().view(np.uint32)):
            failed.append("entries:" + case["name"])

    for (M, K, N) in [(3, 1, 5), (4, 7, 2), (2, 96, 3)]:
        C, S = lib.gemm(np.ones((M, K), np.float32), np.ones((K, N), np.float32))
        if not (np.all(C == np.float32(K)) and np.all(S == K)):
            failed.append(f"ones:{M}x{K}x{N}")

    C, _ = lib.gemm(np.zeros((3, 0), np.float32), np.zeros((0, 4), np.float32))
    if not np.all(C.view(np.uint32) == 0):
        failed.append("empty_sum")

    for case in GENERAL:
        out, S = run_case(lib, case)
        if not case_matches(out, case["Cout"]) or not np.isfinite(S).all():
            failed.append("general:" + case["name"])

    rng = np.random.default_rng(3)
    for (M, K, N) in [(3, 5, 2), (7, 4, 9)]:
        Ai = rng.integers(-16, 17, size=(M, K))
        Bi = rng.integers(-16, 17, size=(K, N))
        if lib.gemm_i64(Ai, Bi).tolist() != _python_int_gemm(Ai.tolist(), Bi.tolist(), M, K, N):
            failed.append(f"i64:{M}x{K}x{N}")
    return failed


def test_real_oracle_passes_every_pin_check():
    oracle.build(force=False)
    assert _pin_failures(oracle.OracleLib(oracle.LIB_PATH)) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} is not unique"
    mutant_src = tmp_path / f"oracle_{name}.c"
    mutant_src.write_text(src.replace(old, new))
    lib_path = oracle.build(force=True, src=str(mutant_src), out=str(tmp_path / f"lib_{name}.so"))
    failures = _pin_failures(oracle.OracleLib(lib_path))
    assert failures, f"mutant {name} survived every pin"

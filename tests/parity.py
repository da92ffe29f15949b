"""Acceptance checks shared by the test files.

Per-element bound for a floating-point result against the oracle:
    |C - C_ref| <= 1e-5 * S + 1e-6,   S = sum_k |A_ik * B_kj|
and raw-bit equality where every partial sum is exact (integer inputs).
"""
import numpy as np

REL = 1e-5
ABS = 1e-6


def within_bound(C, C_ref, S):
    C = np.asarray(C, np.float64)
    C_ref = np.asarray(C_ref, np.float64)
    err = np.abs(C - C_ref)
    bound = REL * np.asarray(S, np.float64) + ABS
    ok = np.isfinite(C) & (err <= bound)
    return ok


def assert_within_bound(C, C_ref, S, what=""):
    ok = within_bound(C, C_ref, S)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        C = np.asarray(C)
        raise AssertionError(
            f"{what}: {bad.shape[0]} of {ok.size} elements outside |C-ref| <= 1e-5*S + 1e-6; "
            f"first at {i}: got {C[i]!r}, ref {np.asarray(C_ref)[i]!r}, S {np.asarray(S)[i]!r}")


def worst_ratio(C, C_ref, S):
    """max over elements of |C - ref| / (1e-5*S + 1e-6); <= 1 passes."""
    err = np.abs(np.asarray(C, np.float64) - np.asarray(C_ref, np.float64))
    return float(np.max(err / (REL * np.asarray(S, np.float64) + ABS))) if err.size else 0.0


def assert_bits_equal(C, C_ref, what=""):
    a = np.ascontiguousarray(C, np.float32).view(np.uint32)
    b = np.ascontiguousarray(C_ref, np.float32).view(np.uint32)
    if not np.array_equal(a, b):
        bad = np.argwhere(a != b)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {bad.shape[0]} of {a.size} elements differ in bits; "
                             f"first at {i}: got {np.asarray(C)[i]!r}, ref {np.asarray(C_ref)[i]!r}")

"""Helpers for the GPU parity tests: device buffers from torch, calls through the C ABI."""
import sys

import numpy as np

import oracle
from fp32_gemm_07_amd import binding
from parity import assert_bits_equal, assert_within_bound

_torch = None


def torch():
    global _torch
    if _torch is None:
        import torch as t
        if not t.cuda.is_available():
            raise RuntimeError("GPU tests need a visible MI355X (torch.cuda.is_available() is False)")
        _torch = t
    return _torch


def say(msg: str) -> None:
    """Name the case on stdout before a GPU step (survives a crashed box)."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def nan_buffer(n: int):
    t = torch()
    return t.full((max(n, 1),), float("nan"), dtype=t.float32, device="cuda:0")


def run(A: np.ndarray, B: np.ndarray, plan=None, stream=None, entry="gemm_f32"):
    """C = A x B on the GPU through the C ABI; C starts as NaN so every output
    must be written. Returns C as a float32 NumPy array."""
    t = torch()
    M, K = A.shape
    K2, N = B.shape
    assert K == K2
    dA, dB = to_dev(A), to_dev(B)
    dC = nan_buffer(M * N)
    s = stream if stream is not None else t.cuda.current_stream()
    h = s.cuda_stream
    if plan is not None:
        need = binding.gemm_f32_plan_workspace_bytes(M, N, K, plan)
        ws = t.empty((max(need // 4, 1),), dtype=t.float32, device="cuda:0")
        binding.gemm_f32_with_plan(dA, dB, dC, M, N, K, plan, ws, need, h)
    elif entry == "gemm_f32_ex":
        need = binding.gemm_f32_workspace_bytes(M, N, K)
        ws = t.empty((max(need // 4, 1),), dtype=t.float32, device="cuda:0")
        binding.gemm_f32_ex(dA, dB, dC, M, N, K, ws, need, h)
    else:
        binding.gemm_f32(dA, dB, dC, M, N, K, h)
    s.synchronize()
    return dC[: M * N].cpu().numpy().reshape(M, N)


# ---------------------------------------------------------------------------
# The general form on strided storage (both sides on the same buffers).

def stored(X: np.ndarray, trans: bool, pad: int):
    """Storage of op = X: X (trans False) or X^T, rows padded with NaN by pad
    floats. Returns (flat storage, ld)."""
    Y = np.ascontiguousarray(X.T if trans else X)
    ld = Y.shape[1] + pad
    buf = np.full((max(Y.shape[0], 1), max(ld, 1)), np.nan, np.float32)
    buf[:Y.shape[0], :Y.shape[1]] = Y
    return buf.ravel(), max(ld, 1)


def run_general(ta, tb, M, N, K, alpha, X, Y, beta, C0, pads=(0, 0, 0), workspace="library"):
    """Both sides on the same strided storage; returns (gpu flat C, oracle flat C, S)."""
    t = torch()
    A, lda = stored(X, ta, pads[0])
    B, ldb = stored(Y, tb, pads[1])
    Cst, ldc = stored(C0, False, pads[2])
    dA, dB, dC = to_dev(A), to_dev(B), to_dev(Cst)
    s = t.cuda.current_stream()
    if workspace == "library":
        binding.gemm_f32_general(ta, tb, M, N, K, alpha, dA, lda, dB, ldb, beta, dC, ldc,
                                 stream=s.cuda_stream)
    else:
        need = binding.gemm_f32_general_workspace_bytes(ta, tb, M, N, K, lda, ldb)
        ws = t.empty((max(need // 4, 1),), dtype=t.float32, device="cuda:0")
        binding.gemm_f32_general(ta, tb, M, N, K, alpha, dA, lda, dB, ldb, beta, dC, ldc, ws,
                                 need, s.cuda_stream)
    s.synchronize()
    got = dC.cpu().numpy()
    ref, S = oracle.gemm_general(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, Cst, ldc)
    return got, ref, S, ldc


def check(got, ref, S, M, N, ldc, what, bits=False):
    g = got.reshape(-1, ldc)
    r = ref.reshape(-1, ldc)
    assert np.isnan(g[:, N:]).all(), f"{what}: padding of C written"
    if bits:
        assert_bits_equal(g[:M, :N], r[:M, :N], what)
    else:
        assert_within_bound(g[:M, :N], r[:M, :N], S, what)

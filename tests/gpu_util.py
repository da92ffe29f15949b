"""Helpers for the GPU parity tests: device buffers from torch, calls through the C ABI."""
import sys

import numpy as np

from fp32_gemm_07_amd import binding

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

"""Work, traffic and peak figures used to place a measured GEMM on the MI355X roofline.

FLOP convention: 2*M*N*K (one multiply and one add per term of each of the
M*N length-K dot products), the convention behind every timing row of the
yekq.top LeetGPU walkthrough's benchmark tables and the 2.147 GFLOP total of
the worked example in the hpc.payai.win lesson 10.

Peaks are MI355X's published figures: 256 compute units at 2.4 GHz, FP32
matrix (MFMA) 157.3 TFLOP/s = 256 CU x 2.4e9 clk/s x 256 FLOP/clk/CU, and
HBM3E 8 TB/s.
"""
from __future__ import annotations

import math

MI355X_CUS = 256
MI355X_CLOCK_GHZ = 2.4
FP32_MFMA_FLOP_PER_CLK_PER_CU = 256
PEAK_FP32_MFMA_TFLOPS = 157.3        # published; = 256 * 2.4 * 256 / 1000 rounded
PEAK_FP32_VALU_TFLOPS = 157.3        # published vector FP32 (packed-FP32 issue)
PEAK_HBM_GBPS = 8000.0               # HBM3E, published


def gemm_flops(M: int, N: int, K: int) -> int:
    """Algorithmic work of C = A x B: 2*M*N*K FLOP (padding is not credited)."""
    return 2 * int(M) * int(N) * int(K)


def compulsory_bytes(M: int, N: int, K: int) -> int:
    """Bytes every implementation must move through HBM at least once:
    read A (M*K) and B (K*N), write C (M*N), all FP32."""
    return 4 * (int(M) * int(K) + int(K) * int(N) + int(M) * int(N))


def splitk_workspace_bytes(M: int, N: int, splits: int) -> int:
    """Extra HBM traffic of a split-K plan: S partial M x N slabs written and read back."""
    return 0 if splits <= 1 else 2 * 4 * int(splits) * int(M) * int(N)


def tiled_read_floats(M: int, N: int, K: int, BM: int, BN: int, BK: int) -> int:
    """Global reads of a block-tiled kernel without cache reuse between blocks:
    each of the ceil(M/BM)*ceil(N/BN) output tiles walks ceil(K/BK) phases and
    loads a BM x BK slice of A and a BK x BN slice of B per phase (the counting
    of the lesson 10 worked example; BM = BN = BK = 1 is the naive kernel that
    reads one A and one B element per multiply-add)."""
    tiles = math.ceil(M / BM) * math.ceil(N / BN)
    phases = math.ceil(K / BK)
    return tiles * phases * (BM * BK + BK * BN)


def arithmetic_intensity(flops: float, nbytes: float) -> float:
    return flops / nbytes if nbytes else math.inf


def ridge_flop_per_byte(peak_tflops: float = PEAK_FP32_MFMA_TFLOPS,
                        peak_gbps: float = PEAK_HBM_GBPS) -> float:
    """FLOP/B at which the compute and bandwidth roofs meet (about 19.7 on MI355X FP32)."""
    return peak_tflops * 1e12 / (peak_gbps * 1e9)

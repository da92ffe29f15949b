"""A NumPy model of block-tiled C = A x B with zero padding and split-K.

It follows the blocked algorithm the pages teach (hpc.payai.win lesson 10,
section 2 and its NumPy simulation section; yekq.top LeetGPU walkthrough,
section v2): every output tile of BM x BN walks the K axis in phases of BK,
each phase loads an A slice and a B slice into a zero-filled on-chip buffer
(elements past M, N or K become 0.0 and so add nothing), multiplies them into
an FP32 accumulator tile, and only the in-range part of the tile is stored.
The split-K extension (not on the pages) gives each of S contiguous K ranges
its own partial tile and then sums the S partials in ascending order. With
a split tail (`tail_round`), tiles are taken in the kernels' tile order
(groups of `group_m` tile rows, column by column inside a group); those of
the whole rounds of `tail_round` tiles are computed over all of K, and only
the tiles of the last, partial round are split.

Test code only: it models the mechanism, it is not the oracle and not the
GPU path.
"""
import math

import numpy as np


def tile_order(tiles_m, tiles_n, group_m=8):
    """(tile row, tile column) of each tile in the kernels' tile order."""
    order = []
    for g0 in range(0, tiles_m, group_m):
        for tn in range(tiles_n):
            order.extend((g0 + i, tn) for i in range(min(group_m, tiles_m - g0)))
    return order


def _tile(A, B, m0, n0, k_lo, k_hi, BM, BN, BK):
    """One output tile over the K range [k_lo, k_hi): zero-filled phases of BK."""
    acc = np.zeros((BM, BN), np.float32)
    for k0 in range(k_lo, k_hi, BK):
        a_buf = np.zeros((BM, BK), np.float32)
        b_buf = np.zeros((BK, BN), np.float32)
        ke = min(k0 + BK, k_hi)
        a_part = A[m0:m0 + BM, k0:ke]
        b_part = B[k0:ke, n0:n0 + BN]
        a_buf[:a_part.shape[0], :a_part.shape[1]] = a_part
        b_buf[:b_part.shape[0], :b_part.shape[1]] = b_part
        acc += a_buf @ b_buf
    return acc


def tiled_gemm(A, B, BM=16, BN=16, BK=16, splits=1, k_chunk=None, tail_round=None, group_m=8):
    A = np.asarray(A, np.float32)
    B = np.asarray(B, np.float32)
    M, K = A.shape
    K2, N = B.shape
    assert K == K2
    if k_chunk is None:
        k_chunk = BK * math.ceil(math.ceil(K / max(splits, 1)) / BK) if K else BK
    n_split = max(1, math.ceil(K / k_chunk)) if K else 1
    order = tile_order(math.ceil(M / BM), math.ceil(N / BN), group_m)
    whole = 0
    if tail_round and n_split > 1:
        whole = len(order) // tail_round * tail_round
        if whole == len(order):   # whole rounds only: nothing is split
            whole, n_split, k_chunk = len(order), 1, K
    C = np.zeros((M, N), np.float32)
    for i, (tm, tn) in enumerate(order):
        m0, n0 = tm * BM, tn * BN
        mh, nh = min(BM, M - m0), min(BN, N - n0)
        if i < whole or n_split == 1:
            C[m0:m0 + mh, n0:n0 + nh] = _tile(A, B, m0, n0, 0, K, BM, BN, BK)[:mh, :nh]
            continue
        total = np.zeros((mh, nh), np.float32)
        for s in range(n_split):
            k_lo, k_hi = s * k_chunk, min(K, (s + 1) * k_chunk)
            total = total + _tile(A, B, m0, n0, k_lo, k_hi, BM, BN, BK)[:mh, :nh]
        C[m0:m0 + mh, n0:n0 + nh] = total
    return C

"""Seeded synthetic inputs for C = A x B (shared by the oracle tests and the GPU tests).

This module holds no arithmetic of the product itself: it only draws the A
and B matrices. Both sides of every parity check take their inputs from here
and from nowhere else.

Recipe (one generator per case, A drawn first, then B):
  - generator: NumPy ``default_rng(seed)`` (PCG64);
  - ``uniform``: ``rng.random(shape, float32) * 2 - 1``; ``rng.random`` yields
    multiples of 2^-24 in [0, 1), so doubling and subtracting one are exact
    and the values are exactly in [-1, 1);
  - ``normal``: ``rng.standard_normal(shape, float32) * (1 / sqrt(K))``; the
    scale is applied in float32 and is exact when K is a power of four
    (1/64 at K = 4096);
  - ``int``: integers drawn uniformly from [-r, r] with
    ``r = min(16, floor(sqrt(2^24 / K)))`` (at least 1), stored as float32;
    every partial sum of any order or grouping is then an integer of
    magnitude <= K * r^2 <= 2^24 and so exact in FP32.

The five standing workloads are the pages' two shapes (1024x512x1024 and the
irregular 1001x513x777 from the yekq.top LeetGPU walkthrough's benchmarks),
a small case, the square 4096^3 roofline case and a long-K case.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    dist: str  # "uniform" | "normal"
    seed: int


WORKLOADS = (
    Workload("small_128x96x112", 128, 96, 112, "uniform", 0),
    Workload("regular_1024x512x1024", 1024, 512, 1024, "uniform", 1),
    Workload("irregular_1001x513x777", 1001, 513, 777, "uniform", 2),
    Workload("square_4096", 4096, 4096, 4096, "normal", 3),
    Workload("longk_512x131072x512", 512, 131072, 512, "uniform", 4),
)
BY_NAME = {w.name: w for w in WORKLOADS}


def int_range(K: int) -> int:
    """Largest |value| r for integer inputs such that K * r^2 <= 2^24 (capped at 16)."""
    if K <= 0:
        return 16
    return max(1, min(16, math.isqrt((1 << 24) // K)))


def draw(M: int, K: int, N: int, dist: str = "uniform", seed: int = 0):
    """Return (A, B) as C-contiguous float32 arrays of shapes (M, K) and (K, N)."""
    rng = np.random.default_rng(seed)
    if dist == "uniform":
        A = rng.random((M, K), dtype=np.float32) * np.float32(2) - np.float32(1)
        B = rng.random((K, N), dtype=np.float32) * np.float32(2) - np.float32(1)
    elif dist == "normal":
        s = np.float32(1.0 / math.sqrt(K)) if K > 0 else np.float32(1)
        A = rng.standard_normal((M, K), dtype=np.float32) * s
        B = rng.standard_normal((K, N), dtype=np.float32) * s
    elif dist == "int":
        r = int_range(K)
        A = rng.integers(-r, r + 1, size=(M, K), dtype=np.int64).astype(np.float32)
        B = rng.integers(-r, r + 1, size=(K, N), dtype=np.int64).astype(np.float32)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return np.ascontiguousarray(A, np.float32), np.ascontiguousarray(B, np.float32)


def draw_workload(w: Workload, integer: bool = False):
    """Inputs of a standing workload; ``integer=True`` gives its small-integer variant."""
    return draw(w.M, w.K, w.N, "int" if integer else w.dist, w.seed)


def sample_indices(M: int, N: int, count: int, seed: int = 12345, tile: int = 32):
    """Output positions to check one by one on large products.

    Covers the four corners, the last row and column, every tile edge
    (rows/cols at multiples of ``tile`` and one before) on a diagonal sweep,
    and ``count`` uniformly random positions. Returns (rows, cols) int64.
    """
    rng = np.random.default_rng(seed)
    r = [0, 0, M - 1, M - 1]
    c = [0, N - 1, 0, N - 1]
    edges_m = sorted({x for t in range(0, M, tile) for x in (t, t - 1) if 0 <= x < M})
    edges_n = sorted({x for t in range(0, N, tile) for x in (t, t - 1) if 0 <= x < N})
    for t, x in enumerate(edges_m):
        r.append(x)
        c.append(edges_n[t % len(edges_n)])
    for t, y in enumerate(edges_n):
        c.append(y)
        r.append(edges_m[(t * 7) % len(edges_m)])
    r.extend(rng.integers(0, M, size=count).tolist())
    c.extend(rng.integers(0, N, size=count).tolist())
    return np.asarray(r, dtype=np.int64), np.asarray(c, dtype=np.int64)


def draw_lesson10_case():
    """The tile-simulation check case of the hpc.payai.win lesson 10 (section
    "NumPy simulation without a GPU"): A is 35x45 and B is 45x25, standard
    normal from NumPy's legacy global seed 42, drawn A first, cast to float32.
    Neither dimension is a multiple of the lesson's tile of 16."""
    rs = np.random.RandomState(42)
    A = rs.randn(35, 45).astype(np.float32)
    B = rs.randn(45, 25).astype(np.float32)
    return A, B

"""Seeded random cases through the C ABI, each against the oracle.

Plain entry (gemm_f32_with_plan): a random kernel of every kind (copy-fed,
register-staged, vector-FMA, ladder), split, split tail (copy-fed kernels)
and shape, on uniform or small-integer inputs (bitwise). General entry: a
random transpose pair, alpha, beta (zeros included), row padding and shape,
K = 0 included. The draws are fixed by the seeds, so every run makes the
same cases; each case is named before it runs.
"""
import numpy as np
import pytest

import gemm_inputs
import oracle
from fp32_gemm_07_amd import binding
from gpu_util import check, run, run_general, say, torch
from parity import assert_bits_equal, assert_within_bound

pytestmark = pytest.mark.gpu

DMA = [k for k in binding.KERNELS if k.startswith("dma")]
KERNEL_NAMES = list(binding.KERNELS)


def plain_cases(n=400, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kname = KERNEL_NAMES[int(rng.integers(len(KERNEL_NAMES)))]
        big = kname in DMA and rng.random() < 0.4
        lo, hi = (1000, 1500) if big else (1, 400)
        M, N = (int(x) for x in rng.integers(lo, hi, 2))
        K = int(rng.integers(1, 700))
        split = int(rng.choice([1, 2, 3, 5, 8]))
        tail = kname in DMA and split > 1 and bool(rng.random() < 0.5)
        dist = "int" if rng.random() < 0.3 else "uniform"
        out.append((i, kname, M, K, N, split, tail, dist))
    return out


def general_cases(n=200, seed=7):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        ta, tb = (int(x) for x in rng.integers(0, 2, 2))
        M, N = (int(x) for x in rng.integers(1, 500, 2))
        K = 0 if rng.random() < 0.05 else int(rng.integers(1, 600))
        alpha = float(rng.choice([1.0, 2.0, -0.5, 0.0]))
        beta = float(rng.choice([0.0, 1.0, -2.0, 0.25]))
        pads = tuple(int(x) for x in rng.integers(0, 6, 3))
        out.append((i, ta, tb, M, K, N, alpha, beta, pads))
    return out


@pytest.fixture(scope="module", autouse=True)
def _setup():
    oracle.build(force=False)
    binding.load()
    torch()


PLAIN = plain_cases()
GENERAL = general_cases()


@pytest.mark.parametrize("i,kname,M,K,N,split,tail,dist", PLAIN,
                         ids=[f"{c[0]}-{c[1]}-{c[2]}x{c[3]}x{c[4]}-S{c[5]}{'t' if c[6] else ''}-{c[7]}"
                              for c in PLAIN])
def test_random_plain_case(i, kname, M, K, N, split, tail, dist):
    say(f"random plain {i}: {kname} {M}x{K}x{N} split {split} tail {tail} {dist}")
    A, B = gemm_inputs.draw(M, K, N, dist, seed=1000 + i)
    C = run(A, B, plan=binding.make_plan(binding.KERNELS[kname], split, tail))
    if dist == "int":
        ref = oracle.gemm_i64(A.astype(np.int64), B.astype(np.int64)).astype(np.float32)
        assert_bits_equal(C, ref, f"case {i}")
    else:
        ref, S = oracle.gemm(A, B)
        assert_within_bound(C, ref, S, f"case {i}")


@pytest.mark.parametrize("i,ta,tb,M,K,N,alpha,beta,pads", GENERAL,
                         ids=[f"{c[0]}-{'TN'[c[1]]}{'TN'[c[2]]}-{c[3]}x{c[4]}x{c[5]}-a{c[6]}b{c[7]}"
                              for c in GENERAL])
def test_random_general_case(i, ta, tb, M, K, N, alpha, beta, pads):
    say(f"random general {i}: {'TN'[ta]}{'TN'[tb]} {M}x{K}x{N} alpha {alpha} beta {beta} "
        f"pads {pads}")
    X, Y = gemm_inputs.draw(M, K, N, "uniform", seed=2000 + i)
    C0 = gemm_inputs.draw(M, N, 1, "uniform", seed=3000 + i)[0]
    got, ref, S, ldc = run_general(ta, tb, M, N, K, alpha, X, Y, beta, C0, pads=pads)
    check(got, ref, S, M, N, ldc, f"general case {i}")

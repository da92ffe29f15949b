"""GPU parity of gemm_f32_general (transposes, row strides, alpha, beta)
against the oracle's general form, through the C ABI.

Operands live inside NaN-filled buffers with padded rows, so a read of
padding turns outputs into NaN and a write past C's rows changes a NaN that
must stay. Floating-point inputs: |C - ref| <= 1e-5 * S + 1e-6 per element,
S = |alpha| sum_k |a b| + |beta c| (the oracle's second output). Small
integers with small integer alpha, beta: raw bits equal.
"""
import numpy as np
import pytest

import gemm_inputs
import oracle
from fp32_gemm_07_amd import binding
from gpu_util import check, nan_buffer, run_general, say, stored, to_dev, torch
from parity import assert_bits_equal, assert_within_bound

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    oracle.build(force=False)
    binding.load()
    torch()


ORDERS = [(0, 0), (1, 0), (0, 1), (1, 1)]
SHAPES = [(1, 1, 1), (33, 17, 31), (65, 129, 63), (300, 513, 260), (257, 40, 255), (128, 96, 112)]
SCALARS = [(1.0, 0.0), (2.0, -0.5), (-1.0, 1.0)]


@pytest.mark.parametrize("ta,tb", ORDERS, ids=["NN", "TN", "NT", "TT"])
@pytest.mark.parametrize("M,K,N", SHAPES, ids=[f"{m}x{k}x{n}" for m, k, n in SHAPES])
@pytest.mark.parametrize("alpha,beta", SCALARS, ids=["a1b0", "a2b-.5", "a-1b1"])
def test_general_parity(ta, tb, M, K, N, alpha, beta):
    say(f"general {'TN'[ta]}{'TN'[tb]} {M}x{K}x{N} alpha {alpha} beta {beta}")
    X, Y = gemm_inputs.draw(M, K, N, "uniform", seed=M + 3 * K + 7 * N + ta + 2 * tb)
    # an M x N draw (the generator's first matrix); NaN when it must not be read
    C0 = gemm_inputs.draw(M, N, 1, "uniform", seed=N)[0] if beta != 0 else \
        np.full((M, N), np.nan, np.float32)
    got, ref, S, ldc = run_general(ta, tb, M, N, K, alpha, X, Y, beta, C0, pads=(3, 5, 2))
    check(got, ref, S, M, N, ldc, f"{ta}{tb} {M}x{K}x{N} {alpha},{beta}")


@pytest.mark.parametrize("ta,tb", ORDERS, ids=["NN", "TN", "NT", "TT"])
@pytest.mark.parametrize("M,K,N", [(32, 2, 32), (65, 129, 63), (300, 513, 260)])
def test_general_integers_bit_exact(ta, tb, M, K, N):
    """Small integers, alpha = 2, beta = -3, integer C: every value exact on
    both sides, so the bits must match (also pins the transposed layouts)."""
    say(f"general int {'TN'[ta]}{'TN'[tb]} {M}x{K}x{N}")
    X, Y = gemm_inputs.draw(M, K, N, "int", seed=K + ta + 2 * tb)
    C0 = gemm_inputs.draw(M, N, 1, "int", seed=5)[0]
    got, ref, S, ldc = run_general(ta, tb, M, N, K, 2.0, X, Y, -3.0, C0, pads=(1, 7, 4))
    check(got, ref, S, M, N, ldc, f"int {ta}{tb}", bits=True)


def test_plain_form_matches_gemm_f32_bitwise():
    say("general NN alpha 1 beta 0 dense == gemm_f32")
    t = torch()
    for w in gemm_inputs.WORKLOADS[:3]:
        X, Y = gemm_inputs.draw_workload(w)
        dA, dB = to_dev(X), to_dev(Y)
        c1, c2 = nan_buffer(w.M * w.N), nan_buffer(w.M * w.N)
        s = t.cuda.current_stream().cuda_stream
        binding.gemm_f32(dA, dB, c1, w.M, w.N, w.K, s)
        binding.gemm_f32_general(0, 0, w.M, w.N, w.K, 1.0, dA, w.K, dB, w.N, 0.0, c2, w.N,
                                 stream=s)
        t.cuda.synchronize()
        assert t.equal(c1.view(t.int32), c2.view(t.int32)), w.name


def test_alpha_zero_reads_neither_operand():
    say("general alpha = 0")
    t = torch()
    M, N = 37, 29
    C0 = gemm_inputs.draw(M, N, 1, "uniform", seed=3)[0]
    dC = to_dev(C0)
    binding.gemm_f32_general(0, 0, M, N, 64, 0.0, None, 64, None, N, 2.5, dC, N)
    t.cuda.synchronize()
    np.testing.assert_array_equal(dC.cpu().numpy().reshape(M, N), np.float32(2.5) * C0)
    binding.gemm_f32_general(1, 1, M, N, 64, 0.0, None, M, None, 64, 0.0, dC, N)
    t.cuda.synchronize()
    assert (dC.view(t.int32) == 0).all()


def test_k_zero_scales_c():
    say("general K = 0")
    t = torch()
    M, N, ldc = 5, 7, 9
    Cst = np.full((M, ldc), np.nan, np.float32)
    Cst[:, :N] = np.arange(M * N, dtype=np.float32).reshape(M, N)
    dC = to_dev(Cst.ravel())
    binding.gemm_f32_general(0, 0, M, N, 0, 1.0, None, 1, None, N, -2.0, dC, ldc)
    t.cuda.synchronize()
    got = dC.cpu().numpy().reshape(M, ldc)
    np.testing.assert_array_equal(got[:, :N], -2.0 * Cst[:, :N])
    assert np.isnan(got[:, N:]).all()


@pytest.mark.parametrize("ta,tb", ORDERS, ids=["NN", "TN", "NT", "TT"])
def test_general_split_k_with_beta_and_strides(ta, tb):
    """A shape the planner splits (256 x 8192 x 256): the reduction applies
    alpha, beta and ldc; caller workspace and library workspace agree bitwise."""
    M, K, N = 256, 8192, 256
    say(f"general split-K {'TN'[ta]}{'TN'[tb]}")
    X, Y = gemm_inputs.draw(M, K, N, "uniform", seed=40 + ta + 2 * tb)
    C0 = gemm_inputs.draw(M, N, 1, "uniform", seed=41)[0]
    g1, ref, S, ldc = run_general(ta, tb, M, N, K, 1.5, X, Y, 0.25, C0, pads=(4, 4, 4))
    g2, _, _, _ = run_general(ta, tb, M, N, K, 1.5, X, Y, 0.25, C0, pads=(4, 4, 4),
                              workspace="caller")
    check(g1, ref, S, M, N, ldc, "split-K general")
    assert np.array_equal(g1.view(np.uint32), g2.view(np.uint32))


@pytest.mark.parametrize("ta,tb", ORDERS, ids=["NN", "TN", "NT", "TT"])
def test_general_large_square(ta, tb):
    """2048 x 1024 x 2048 through the planner's large-tile kernels, full check."""
    M, K, N = 2048, 1024, 2048
    say(f"general large {'TN'[ta]}{'TN'[tb]}")
    X, Y = gemm_inputs.draw(M, K, N, "normal", seed=50 + ta + 2 * tb)
    C0 = np.full((M, N), np.nan, np.float32)
    got, ref, S, ldc = run_general(ta, tb, M, N, K, 1.0, X, Y, 0.0, C0, pads=(0, 0, 0))
    check(got, ref, S, M, N, ldc, "large general")


def test_general_k_passes_for_long_strided_rows():
    """B (not transposed) with rows 4M floats apart: one K range of 200 would
    span more than 2^31 bytes of copy offsets, so the call runs in K passes,
    each after the first accumulating into C."""
    t = torch()
    M, K, N = 64, 200, 96
    ldb = 1 << 22
    say(f"general K passes ldb {ldb}")
    X, Y = gemm_inputs.draw(M, K, N, "uniform", seed=60)
    dA = to_dev(X)
    dBbig = t.full((K, ldb), float("nan"), dtype=t.float32, device="cuda:0")
    dBbig[:, :N] = to_dev(Y)
    C0 = gemm_inputs.draw(M, N, 1, "uniform", seed=61)[0]
    dC = to_dev(C0)
    binding.gemm_f32_general(0, 0, M, N, K, 1.0, dA, K, dBbig, ldb, 0.5, dC, N)
    t.cuda.synchronize()
    got = dC.cpu().numpy().reshape(M, N)
    del dBbig
    ref, S = oracle.gemm_general(0, 0, M, N, K, 1.0, X, K, Y, N, 0.5, C0, N)
    assert_within_bound(got, ref.reshape(M, N), S, "K passes")


@pytest.mark.parametrize("ta,tb", ORDERS, ids=["NN", "TN", "NT", "TT"])
def test_general_guard_bands_misaligned(ta, tb):
    """A, B and C, each shifted by one float (4-byte aligned only) and with
    padded rows, inside one NaN-filled buffer with NaN guards around each:
    a read outside an operand turns outputs into NaN, a write outside C's
    M x N elements changes a NaN that must stay."""
    t = torch()
    M, K, N = 97, 53, 71
    say(f"general guard bands {'TN'[ta]}{'TN'[tb]}")
    X, Y = gemm_inputs.draw(M, K, N, "uniform", seed=70 + ta + 2 * tb)
    C0 = gemm_inputs.draw(M, N, 1, "uniform", seed=71)[0]
    A, lda = stored(X, ta, 3)
    B, ldb = stored(Y, tb, 2)
    Cs, ldc = stored(C0, False, 5)
    g = 257
    offA = g
    offB = offA + A.size + g
    offC = offB + B.size + g
    total = offC + Cs.size + g
    host = np.full(total, np.nan, np.float32)
    host[offA:offA + A.size] = A
    host[offB:offB + B.size] = B
    host[offC:offC + Cs.size] = Cs
    buf = to_dev(host)
    base = buf.data_ptr()
    binding.gemm_f32_general(ta, tb, M, N, K, 1.25, base + 4 * offA, lda, base + 4 * offB, ldb,
                             -0.75, base + 4 * offC, ldc)
    t.cuda.synchronize()
    out = buf.cpu().numpy()
    ref, S = oracle.gemm_general(ta, tb, M, N, K, 1.25, A, lda, B, ldb, -0.75, Cs, ldc)
    check(out[offC:offC + Cs.size], ref, S, M, N, ldc, "guarded general")
    guards = np.concatenate([out[:offA], out[offA + A.size:offB], out[offB + B.size:offC],
                             out[offC + Cs.size:]])
    assert np.isnan(guards).all()
    np.testing.assert_array_equal(out[offA:offA + A.size], A)
    np.testing.assert_array_equal(out[offB:offB + B.size], B)


_FULL = {}


def _square_operands():
    """op(A), op(B) of the 4096^3 general-form cases and the oracle's product,
    computed once for the three transposed orders."""
    if "square" not in _FULL:
        X, Y = gemm_inputs.draw(4096, 4096, 4096, "normal", seed=80)
        _FULL["square"] = (X, Y) + oracle.gemm(X, Y)
    return _FULL["square"]


@pytest.mark.parametrize("ta,tb", [(1, 0), (0, 1), (1, 1)], ids=["TN", "NT", "TT"])
def test_general_full_size_every_element(ta, tb):
    """4096^3 in the transposed orders through the planner's 256 x 256 kernel:
    every output against the oracle's product of op(A) and op(B) (alpha = 1,
    beta = 0 is the plain product, whatever the storage order)."""
    t = torch()
    M = N = K = 4096
    say(f"general full size {'TN'[ta]}{'TN'[tb]}")
    X, Y, C_ref, S = _square_operands()
    dA = to_dev(np.ascontiguousarray(X.T) if ta else X)
    dB = to_dev(np.ascontiguousarray(Y.T) if tb else Y)
    dC = nan_buffer(M * N)
    binding.gemm_f32_general(ta, tb, M, N, K, 1.0, dA, M if ta else K, dB, K if tb else N, 0.0,
                             dC, N)
    t.cuda.synchronize()
    C = dC.cpu().numpy().reshape(M, N)
    del dA, dB, dC
    assert_within_bound(C, C_ref, S, "general 4096^3")


@pytest.mark.parametrize("ta,tb", ORDERS, ids=["NN", "TN", "NT", "TT"])
def test_general_large_tile_ragged(ta, tb):
    """A ragged shape whose plan is the 256 x 256 kernel (its transposed-A
    form reads interleaved rows): every output against the oracle, with
    alpha, beta and padded strides."""
    M, K, N = 4001, 419, 3999
    plan = binding.gemm_f32_plan(M, N, K)
    assert binding.gemm_kernel_name(plan.kernel).startswith("dma_mfma32_f32_256x256")
    say(f"general 256-tile ragged {'TN'[ta]}{'TN'[tb]}")
    X, Y = gemm_inputs.draw(M, K, N, "uniform", seed=90 + ta + 2 * tb)
    C0 = gemm_inputs.draw(M, N, 1, "uniform", seed=91)[0]
    got, ref, S, ldc = run_general(ta, tb, M, N, K, 1.5, X, Y, -0.5, C0, pads=(2, 3, 1))
    check(got, ref, S, M, N, ldc, "256-tile ragged general")


GENERAL_TAILS = [((1100, 777, 1000), 0, 0, (0, 0, 0)), ((1100, 777, 1000), 1, 0, (2, 3, 1)),
                 ((1100, 777, 1000), 0, 1, (0, 0, 4)), ((1100, 777, 1000), 1, 1, (1, 1, 2)),
                 ((1792, 1792, 1792), 0, 0, (0, 0, 0)), ((1792, 1792, 1792), 0, 0, (3, 1, 2)),
                 ((1792, 1792, 1792), 1, 0, (1, 2, 3)), ((1792, 1792, 1792), 0, 1, (0, 0, 0)),
                 ((1792, 1792, 1792), 1, 1, (2, 0, 1))]


@pytest.mark.parametrize("shape,ta,tb,pads", GENERAL_TAILS,
                         ids=[f"{m}x{k}x{n}-{'TN'[a]}{'TN'[b]}-{''.join(map(str, p))}"
                              for (m, k, n), a, b, p in GENERAL_TAILS])
def test_general_split_tail(shape, ta, tb, pads):
    """Shapes whose plans split only the last round of tiles (64 x 64 tiles at
    1100 x 777 x 1000, 96 x 96 at 1792^3, each in every storage order): the reduction of
    the split tiles applies alpha, beta and ldc (row strides that are and are
    not multiples of 4), the whole tiles are stored directly; every output
    against the oracle."""
    M, K, N = shape
    assert binding.gemm_f32_plan(M, N, K).split_tail == 1
    say(f"general split tail {M}x{K}x{N} {'TN'[ta]}{'TN'[tb]} pads {pads}")
    X, Y = gemm_inputs.draw(M, K, N, "uniform", seed=100 + ta + 2 * tb)
    C0 = gemm_inputs.draw(M, N, 1, "uniform", seed=101)[0]
    got, ref, S, ldc = run_general(ta, tb, M, N, K, 1.5, X, Y, -0.5, C0, pads=pads)
    check(got, ref, S, M, N, ldc, "split tail general")


# Shapes the planner gives 96 x 96 tiles, none split: 1536^3 (16 x 16 tiles,
# one per CU), ragged M and N with K % 32 = 7 (1531 x 999 x 1529: rows of
# A^T and B not 16-byte multiples) and a last K step of one element
# (1529 x 4097 x 1531).
TILES_96 = [((1536, 1536, 1536), (0, 0, 0)), ((1536, 1536, 1536), (3, 1, 2)),
            ((1531, 999, 1529), (2, 3, 1)), ((1529, 4097, 1531), (1, 0, 3))]


@pytest.mark.parametrize("ta,tb", ORDERS, ids=["NN", "TN", "NT", "TT"])
@pytest.mark.parametrize("shape,pads", TILES_96,
                         ids=[f"{m}x{k}x{n}-{''.join(map(str, p))}" for (m, k, n), p in TILES_96])
def test_general_96_tiles(ta, tb, shape, pads):
    """The 96 x 96 kernel (16 x 16 blocks; M- and N-contiguous operands
    stored as 32-column panels, K-contiguous ones as swizzled rows) in every
    storage order: alpha, beta and row strides through its own stores; every
    output against the oracle."""
    M, K, N = shape
    p = binding.gemm_f32_plan(M, N, K)
    assert binding.gemm_kernel_name(p.kernel) == "dma_mfma16_f32_96x96x32_w4_s3" and p.split_k == 1
    say(f"general 96 x 96 tiles {'TN'[ta]}{'TN'[tb]} {M}x{K}x{N} pads {pads}")
    X, Y = gemm_inputs.draw(M, K, N, "uniform", seed=111 + ta + 2 * tb + K)
    C0 = gemm_inputs.draw(M, N, 1, "uniform", seed=112)[0]
    got, ref, S, ldc = run_general(ta, tb, M, N, K, 1.5, X, Y, -0.5, C0, pads=pads)
    check(got, ref, S, M, N, ldc, f"96 x 96 general {ta}{tb} {M}x{K}x{N}")


@pytest.mark.parametrize("ta,tb", ORDERS, ids=["NN", "TN", "NT", "TT"])
def test_general_96_tiles_integers_bit_exact(ta, tb):
    """Small integers through the 96 x 96 kernel in every storage order
    (1531 x 999 x 1529, alpha = 2, beta = -3): every value exact on both
    sides, so the bits must match; pins which k each lane group reads from
    the panels and swizzled rows."""
    M, K, N = 1531, 999, 1529
    p = binding.gemm_f32_plan(M, N, K)
    assert binding.gemm_kernel_name(p.kernel) == "dma_mfma16_f32_96x96x32_w4_s3"
    say(f"general 96 x 96 int {'TN'[ta]}{'TN'[tb]}")
    X, Y = gemm_inputs.draw(M, K, N, "int", seed=120 + ta + 2 * tb)
    C0 = gemm_inputs.draw(M, N, 1, "int", seed=121)[0]
    got, ref, S, ldc = run_general(ta, tb, M, N, K, 2.0, X, Y, -3.0, C0, pads=(1, 2, 3))
    check(got, ref, S, M, N, ldc, f"96 x 96 int {ta}{tb}", bits=True)


# A last K step of 1 to 4 elements in the planner's plans: the kernels with few
# accumulators per wave read it into registers instead of staging it in LDS.
# Shapes whose plans put it in every variant the general form reaches: a
# 16-way split (last range only), a split tail (the whole tiles and the last
# range of the split ones), the 8-wave 128 x 128 kernel whole and with a split
# tail; every storage order, alpha, beta and padded rows.
SHORT_STEP = [((256, 8193, 256), "dma_mfma32_f32_64x64x16_w4_s3", 16, 0),
              ((1100, 785, 1000), "dma_mfma32_f32_64x64x16_w4_s3", 2, 1),
              ((2048, 2049, 2048), "dma_mfma32_f32_128x128x16_w8_s3", 1, 0),
              ((3200, 3201, 3200), "dma_mfma32_f32_128x128x16_w8_s3", 2, 1)]


@pytest.mark.parametrize("ta,tb", ORDERS, ids=["NN", "TN", "NT", "TT"])
@pytest.mark.parametrize("shape,kernel,split,tail", SHORT_STEP,
                         ids=[f"{m}x{k}x{n}" for (m, k, n), _, _, _ in SHORT_STEP])
def test_general_short_last_step(ta, tb, shape, kernel, split, tail):
    M, K, N = shape
    p = binding.gemm_f32_plan(M, N, K)
    assert (binding.gemm_kernel_name(p.kernel), p.split_k, p.split_tail) == (kernel, split, tail)
    say(f"general short last step {'TN'[ta]}{'TN'[tb]} {M}x{K}x{N}")
    X, Y = gemm_inputs.draw(M, K, N, "uniform", seed=K + ta + 2 * tb)
    C0 = gemm_inputs.draw(M, N, 1, "uniform", seed=K + 1)[0]
    got, ref, S, ldc = run_general(ta, tb, M, N, K, 1.5, X, Y, -0.5, C0, pads=(3, 1, 2))
    check(got, ref, S, M, N, ldc, f"short last step {ta}{tb} {M}x{K}x{N}")


@pytest.mark.parametrize("ta,tb", ORDERS, ids=["NN", "TN", "NT", "TT"])
@pytest.mark.parametrize("shape,kernel,split,tail", SHORT_STEP[:3],
                         ids=[f"{m}x{k}x{n}" for (m, k, n), _, _, _ in SHORT_STEP[:3]])
def test_general_short_last_step_integers_bit_exact(ta, tb, shape, kernel, split, tail):
    M, K, N = shape
    say(f"general short last step int {'TN'[ta]}{'TN'[tb]} {M}x{K}x{N}")
    X, Y = gemm_inputs.draw(M, K, N, "int", seed=K + 3 + ta + 2 * tb)
    C0 = gemm_inputs.draw(M, N, 1, "int", seed=7)[0]
    got, ref, S, ldc = run_general(ta, tb, M, N, K, 2.0, X, Y, -3.0, C0, pads=(1, 2, 3))
    check(got, ref, S, M, N, ldc, f"short last step int {ta}{tb} {M}x{K}x{N}", bits=True)


@pytest.mark.parametrize("ta,tb,pads", [(0, 0, (0, 0, 0)), (0, 0, (3, 1, 2)), (1, 0, (2, 3, 1)),
                                        (0, 1, (0, 0, 4)), (1, 1, (1, 1, 2))],
                         ids=["NN", "NN-padded", "TN", "NT", "TT"])
def test_general_short_k_large_output(ta, tb, pads):
    """4096 x 16 x 4096: the plain product's plan is the 4-wave 128 x 128
    kernel (store-bound regime); the general form takes it in every storage
    order, with alpha, beta and row strides. Every output against the
    oracle."""
    M = N = 4096
    K = 16
    assert binding.gemm_f32_plan(M, N, K).kernel == binding.GEMM_KERNEL_DMA32_128x128_W4
    say(f"general short K {'TN'[ta]}{'TN'[tb]} pads {pads}")
    X, Y = gemm_inputs.draw(M, K, N, "uniform", seed=120 + ta + 2 * tb)
    C0 = gemm_inputs.draw(M, N, 1, "uniform", seed=121)[0]
    got, ref, S, ldc = run_general(ta, tb, M, N, K, 0.75, X, Y, 2.0, C0, pads=pads)
    check(got, ref, S, M, N, ldc, "short K general")


# Short K over large ragged outputs, planned to the 4-wave 128 x 128 kernel:
# edge tiles on both sides (M, N not multiples of 128), a K range shorter
# than one step (15), one step and one element (17), one step and 15 (31).
SHORT_K_RAGGED = [((4001, 17, 3999), (1, 2, 3)), ((3999, 15, 4001), (0, 0, 0)),
                  ((4097, 31, 4095), (3, 1, 2))]


@pytest.mark.parametrize("ta,tb", ORDERS, ids=["NN", "TN", "NT", "TT"])
@pytest.mark.parametrize("shape,pads", SHORT_K_RAGGED,
                         ids=[f"{m}x{k}x{n}" for (m, k, n), _ in SHORT_K_RAGGED])
def test_general_short_k_ragged(ta, tb, shape, pads):
    """The 4-wave 128 x 128 kernel in every storage order on ragged short-K
    products, alpha and beta, padded rows: every output against the oracle."""
    M, K, N = shape
    assert binding.gemm_f32_plan(M, N, K).kernel == binding.GEMM_KERNEL_DMA32_128x128_W4
    say(f"general short K ragged {'TN'[ta]}{'TN'[tb]} {M}x{K}x{N}")
    X, Y = gemm_inputs.draw(M, K, N, "uniform", seed=130 + K + ta + 2 * tb)
    C0 = gemm_inputs.draw(M, N, 1, "uniform", seed=131)[0]
    got, ref, S, ldc = run_general(ta, tb, M, N, K, 0.75, X, Y, 2.0, C0, pads=pads)
    check(got, ref, S, M, N, ldc, f"short K ragged {ta}{tb} {M}x{K}x{N}")


@pytest.mark.parametrize("ta,tb", ORDERS, ids=["NN", "TN", "NT", "TT"])
def test_general_short_k_ragged_integers_bit_exact(ta, tb):
    """Small integers through the 4-wave 128 x 128 kernel in every storage
    order (4001 x 17 x 3999, alpha = 2, beta = -3): bit for bit, which pins
    which k each lane reads from the transposed layouts and the zeroed tail."""
    M, K, N = 4001, 17, 3999
    assert binding.gemm_f32_plan(M, N, K).kernel == binding.GEMM_KERNEL_DMA32_128x128_W4
    say(f"general short K ragged int {'TN'[ta]}{'TN'[tb]}")
    X, Y = gemm_inputs.draw(M, K, N, "int", seed=140 + ta + 2 * tb)
    C0 = gemm_inputs.draw(M, N, 1, "int", seed=141)[0]
    got, ref, S, ldc = run_general(ta, tb, M, N, K, 2.0, X, Y, -3.0, C0, pads=(2, 1, 1))
    check(got, ref, S, M, N, ldc, f"short K ragged int {ta}{tb}", bits=True)


# IEEE special values through the transposed layouts of the 96 x 96 kernel
# (1531 x 999 x 1529) and the 4-wave 128 x 128 kernel (4001 x 17 x 3999):
# every output is a sum of products over all of K, so neither the panels, the
# swizzled rows, the zero fill of the edges nor the K tail may add a NaN or
# hide one.
SPECIAL_GENERAL = [((1531, 999, 1529), 700, 333, 901, 1000, [5, 1500]),
                   ((4001, 17, 3999), 2100, 3, 16, 3001, [7, 4000])]


@pytest.mark.parametrize("ta,tb", ORDERS[1:], ids=["TN", "NT", "TT"])
@pytest.mark.parametrize("case", SPECIAL_GENERAL, ids=[f"{m}x{k}x{n}" for (m, k, n), *_ in SPECIAL_GENERAL])
def test_general_special_values(ta, tb, case):
    """A NaN at op(A)[i0, k0] makes row i0 NaN; a +Inf at op(B)[k1, j1] makes
    column j1 +-Inf by the sign of op(A)[i, k1], NaN where that is 0; the
    rest finite and within the bound of the oracle's general form."""
    (M, K, N), i0, k0, k1, j1, zeros = case
    assert binding.gemm_kernel_name(binding.gemm_f32_plan(M, N, K).kernel) in (
        "dma_mfma16_f32_96x96x32_w4_s3", "dma_mfma32_f32_128x128x16_w4_s4")
    say(f"general special values {'TN'[ta]}{'TN'[tb]} {M}x{K}x{N}")
    X, Y = gemm_inputs.draw(M, K, N, "uniform", seed=150 + ta + 2 * tb)
    X[i0, k0] = np.nan
    Y[k1, j1] = np.inf
    X[zeros, k1] = 0.0
    C0 = np.full((M, N), np.nan, np.float32)
    got, ref, S, ldc = run_general(ta, tb, M, N, K, 1.0, X, Y, 0.0, C0, pads=(1, 2, 3))
    C = got.reshape(-1, ldc)[:M, :N]
    want_nan = np.zeros((M, N), dtype=bool)
    want_nan[i0, :] = True
    want_nan[zeros, j1] = True
    assert np.array_equal(np.isnan(C), want_nan), "NaN pattern"
    rows = np.delete(np.arange(M), [i0, *zeros])
    assert np.array_equal(C[rows, j1], np.where(X[rows, k1] > 0, np.inf, -np.inf).astype(np.float32))
    R = ref.reshape(-1, ldc)[:M, :N]
    assert np.array_equal(np.isnan(R), want_nan)
    fin = np.isfinite(R)
    fin[:, j1] = False
    assert fin.sum() == (M - 1) * (N - 1)
    assert np.isfinite(C[fin]).all()
    err = np.abs(C[fin].astype(np.float64) - R[fin])
    assert (err <= 1e-5 * S.reshape(M, N)[fin] + 1e-6).all(), f"worst {err.max()}"
    assert np.isnan(got.reshape(-1, ldc)[:, N:]).all(), "padding of C written"


@pytest.mark.parametrize("ta,tb", ORDERS, ids=["NN", "TN", "NT", "TT"])
def test_column_major_through_swapped_operands(ta, tb):
    """The column-major recipe of the header: A, B, C stored column-major
    (padded leading dimensions), the call made with the operands and their
    transpose flags swapped and M, N exchanged; the result, read back as
    column-major, against the oracle's row-major alpha * op(A) op(B) + beta * C."""
    t = torch()
    M, K, N = 97, 53, 71
    say(f"column-major {'TN'[ta]}{'TN'[tb]}")
    X, Y = gemm_inputs.draw(M, K, N, "uniform", seed=110 + ta + 2 * tb)   # op(A), op(B)
    C0 = gemm_inputs.draw(M, N, 1, "uniform", seed=111)[0]
    # Column-major storage is row-major storage of the transpose: op(A) = A
    # (M x K column-major) is stored as X^T row-major; op(A) = A^T means A is
    # K x M column-major, i.e. X row-major. Likewise for B; C is X-like (M x N
    # column-major = C^T row-major).
    A, lda = stored(X, ta == 0, 2)
    B, ldb = stored(Y, tb == 0, 3)
    Cs, ldc = stored(C0.T, False, 1)
    dA, dB, dC = to_dev(A), to_dev(B), to_dev(Cs)
    binding.gemm_f32_general(tb, ta, N, M, K, 1.5, dB, ldb, dA, lda, -0.5, dC, ldc)
    t.cuda.synchronize()
    got = dC.cpu().numpy().reshape(-1, ldc)
    assert np.isnan(got[:, M:]).all(), "padding of C written"
    ref, S = oracle.gemm_general(0, 0, M, N, K, 1.5, X, K, Y, N, -0.5, C0, N)
    assert_within_bound(got[:N, :M].T, ref.reshape(M, N), S.reshape(M, N), "column-major")


def _long_k_case():
    """op(A), op(B), C0 of the long-K general-form cases and the oracle's
    alpha * op(A) op(B) + beta * C0 (alpha = 1.5, beta = -0.5), computed once.
    The oracle is given op(B) stored transposed (N x K), so both of its inner
    reads run along K; its result is a function of op(A), op(B) and C alone,
    whatever the storage (the general form's pins tie every storage order to
    the plain product)."""
    if "long_k" not in _FULL:
        M, K, N = 512, 131072, 512
        X, Y = gemm_inputs.draw(M, K, N, "uniform", seed=120)
        C0 = gemm_inputs.draw(M, N, 1, "uniform", seed=121)[0]
        ref, S = oracle.gemm_general(0, 1, M, N, K, 1.5, X, K, np.ascontiguousarray(Y.T), K, -0.5,
                                     C0, N)
        _FULL["long_k"] = (X, Y, C0, ref.reshape(M, N), S)
    return _FULL["long_k"]


@pytest.mark.parametrize("ta,tb", [(1, 0), (0, 1), (1, 1)], ids=["TN", "NT", "TT"])
def test_general_long_k_full_size_every_element(ta, tb):
    """512 x 131072 x 512 (the long-K workload, K split 16 ways) in the
    transposed orders, alpha = 1.5, beta = -0.5: every output against the
    oracle's general form."""
    t = torch()
    M, K, N = 512, 131072, 512
    say(f"general long K {'TN'[ta]}{'TN'[tb]}")
    X, Y, C0, ref, S = _long_k_case()
    dA = to_dev(np.ascontiguousarray(X.T) if ta else X)
    dB = to_dev(np.ascontiguousarray(Y.T) if tb else Y)
    dC = to_dev(C0)
    binding.gemm_f32_general(ta, tb, M, N, K, 1.5, dA, M if ta else K, dB, K if tb else N, -0.5,
                             dC, N)
    t.cuda.synchronize()
    C = dC.cpu().numpy().reshape(M, N)
    assert_within_bound(C, ref, S, "general long K")


# ---------------------------------------------------------------------------
# The epilogue's rounding, as the header states it: beta * c is rounded to
# FP32 first, then alpha * sum + fl(beta * c) is one fused multiply-add. The
# operands make every sum exact (A has one nonzero column, B is all ones), so
# each output's bits depend on the epilogue alone, and many outputs differ
# between that form and a single rounding of alpha * sum + beta * c (the
# oracle's reading, within the tolerance of either).

EPILOGUE_CASES = [(64, 1, 64, "direct store"), (128, 16384, 128, "split-K reduction"),
                  (1792, 1792, 1792, "split tail: direct store and tail reduction")]


def epilogue_operands(M, K, N, seed):
    rng = np.random.default_rng(seed)
    alpha, beta = np.float32(1.5), np.float32(float.fromhex("0x1.9471f8p+0"))
    s = rng.uniform(0.5, 2.0, M).astype(np.float32)
    X = np.zeros((M, K), np.float32)
    X[:, 0] = s
    Y = np.ones((K, N), np.float32)
    C0 = rng.uniform(0.5, 2.0, (M, N)).astype(np.float32)
    # Sums are exact: sum[i, j] = s[i]. In double, alpha * s, beta * c and each
    # of the sums below are exact (operands in [0.5, 2), 48-bit products), so
    # casting to FP32 rounds once.
    a_s = np.float64(alpha) * s.astype(np.float64)[:, None]
    bc32 = (beta * C0).astype(np.float32)                        # FP32 product, rounded
    fused = (a_s + bc32.astype(np.float64)).astype(np.float32)
    single = (a_s + np.float64(beta) * C0.astype(np.float64)).astype(np.float32)
    return alpha, beta, X, Y, C0, fused, single


@pytest.mark.parametrize("M,K,N,path", EPILOGUE_CASES, ids=[c[3] for c in EPILOGUE_CASES])
def test_general_epilogue_rounds_beta_c_then_fuses(M, K, N, path):
    t = torch()
    plan = binding.gemm_f32_plan(M, N, K)
    say(f"epilogue rounding {M}x{K}x{N} ({path}) plan {plan}")
    if K > 1:
        assert plan.split_k > 1 and plan.split_tail == (1 if M == 1792 else 0)
    alpha, beta, X, Y, C0, fused, single = epilogue_operands(M, K, N, seed=M + K)
    differ = fused.view(np.uint32) != single.view(np.uint32)
    assert differ.mean() > 0.01, "operands do not tell the two roundings apart"
    dA, dB, dC = to_dev(X), to_dev(Y), to_dev(C0)
    binding.gemm_f32_general(0, 0, M, N, K, float(alpha), dA, K, dB, N, float(beta), dC, N)
    t.cuda.synchronize()
    got = dC.cpu().numpy()
    assert_bits_equal(got, fused, f"fmaf(alpha, sum, fl(beta * c)), {path}")
    # the oracle (one rounding) accepts both, within the bound
    ref, S = oracle.gemm_general(0, 0, M, N, K, float(alpha), X, K, Y, N, float(beta), C0, N)
    assert_bits_equal(ref.reshape(M, N), single, "oracle: one rounding")
    assert_within_bound(got, ref.reshape(M, N), S, path)

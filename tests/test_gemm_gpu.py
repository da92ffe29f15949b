"""GPU parity of libgemm against the CPU oracle, through the C ABI.

Floating-point inputs: every element within |C - ref| <= 1e-5 * S + 1e-6,
S = sum_k |A_ik B_kj| (the oracle's second output). Integer inputs whose every
partial sum is exact in FP32: raw bits equal. C starts as NaN before every
call, so an output that is never written fails.
"""
import numpy as np
import pytest

import gemm_inputs
import oracle
from fp32_gemm_07_amd import binding
from gpu_util import nan_buffer, run, say, to_dev, torch
from parity import assert_bits_equal, assert_within_bound

pytestmark = pytest.mark.gpu

SMALL = [w for w in gemm_inputs.WORKLOADS if w.M * w.N * w.K <= 1 << 30]
LARGE = [w for w in gemm_inputs.WORKLOADS if w.M * w.N * w.K > 1 << 30]


@pytest.fixture(scope="module", autouse=True)
def _setup():
    oracle.build(force=False)
    binding.load()
    torch()


# ---------------------------------------------------------------------------
# Standing workloads, planner's choice (the launch configuration the bench times).

@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_workload_full_parity(w):
    say(f"workload {w.name} plan {binding.gemm_f32_plan(w.M, w.N, w.K)}")
    A, B = gemm_inputs.draw_workload(w)
    C = run(A, B)
    C_ref, S = oracle.gemm(A, B)
    assert_within_bound(C, C_ref, S, w.name)


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_workload_small_integers_bit_exact(w):
    say(f"workload {w.name} (integers)")
    A, B = gemm_inputs.draw_workload(w, integer=True)
    C = run(A, B)
    C_ref = oracle.gemm_i64(A.astype(np.int64), B.astype(np.int64)).astype(np.float32)
    assert_bits_equal(C, C_ref, w.name + " int")


@pytest.mark.parametrize("w", LARGE, ids=[w.name for w in LARGE])
def test_workload_full_size_every_element(w):
    """Full size, planner's plan (the launch configuration the bench times):
    every output against the oracle's full product, and a rerun bit-identical
    (fixed split-K order)."""
    t = torch()
    say(f"workload {w.name} plan {binding.gemm_f32_plan(w.M, w.N, w.K)}")
    A, B = gemm_inputs.draw_workload(w)
    dA, dB = to_dev(A), to_dev(B)
    dC = nan_buffer(w.M * w.N)
    s = t.cuda.current_stream()
    binding.gemm_f32(dA, dB, dC, w.M, w.N, w.K, s.cuda_stream)
    s.synchronize()
    C = dC.cpu().numpy().reshape(w.M, w.N)
    dC2 = nan_buffer(w.M * w.N)
    binding.gemm_f32(dA, dB, dC2, w.M, w.N, w.K, s.cuda_stream)
    s.synchronize()
    assert t.equal(dC.view(t.int32), dC2.view(t.int32))
    del dA, dB, dC, dC2
    C_ref, S = oracle.gemm(A, B)
    assert_within_bound(C, C_ref, S, w.name)


@pytest.mark.parametrize("w", LARGE, ids=[w.name for w in LARGE])
def test_workload_full_size_integers_bit_exact(w):
    """Full size on small-integer inputs: every output equal in bits to the
    exact integer product."""
    say(f"workload {w.name} (integers, every element)")
    A, B = gemm_inputs.draw_workload(w, integer=True)
    C = run(A, B)
    C_ref = oracle.gemm_i64(A.astype(np.int64), B.astype(np.int64)).astype(np.float32)
    assert_bits_equal(C, C_ref, w.name + " int")


# ---------------------------------------------------------------------------
# Every kernel, ragged shapes spanning several tiles, with and without split-K.

KERNELS = list(binding.KERNELS.items())
RAGGED = [(1, 1, 1), (32, 2, 32), (33, 17, 31), (64, 16, 64), (65, 129, 63), (127, 40, 129),
          (257, 33, 255), (300, 513, 260), (128, 96, 112), (512, 64, 513)]


@pytest.mark.parametrize("kname,kid", KERNELS, ids=[k for k, _ in KERNELS])
@pytest.mark.parametrize("M,K,N", RAGGED, ids=[f"{m}x{k}x{n}" for m, k, n in RAGGED])
@pytest.mark.parametrize("split", [1, 3])
def test_kernel_ragged_parity(kname, kid, M, K, N, split):
    say(f"kernel {kname} {M}x{K}x{N} split {split}")
    A, B = gemm_inputs.draw(M, K, N, "uniform", seed=M * 7 + K * 3 + N)
    C = run(A, B, plan=binding.make_plan(kid, split))
    C_ref, S = oracle.gemm(A, B)
    assert_within_bound(C, C_ref, S, f"{kname} {M}x{K}x{N}/{split}")


@pytest.mark.parametrize("kname,kid", KERNELS, ids=[k for k, _ in KERNELS])
@pytest.mark.parametrize("M,K,N", [(32, 2, 32), (65, 129, 63), (300, 513, 260), (256, 64, 256)])
@pytest.mark.parametrize("split", [1, 4])
def test_kernel_integers_bit_exact(kname, kid, M, K, N, split):
    """Integer inputs pin the MFMA operand and accumulator lane layouts: a
    32x2 by 2x32 product is exactly one v_mfma_f32_32x32x2_f32."""
    say(f"kernel {kname} int {M}x{K}x{N} split {split}")
    A, B = gemm_inputs.draw(M, K, N, "int", seed=K)
    C = run(A, B, plan=binding.make_plan(kid, split))
    C_ref = oracle.gemm_i64(A.astype(np.int64), B.astype(np.int64)).astype(np.float32)
    assert_bits_equal(C, C_ref, f"{kname} int {M}x{K}x{N}/{split}")


# ---------------------------------------------------------------------------
# Split tail: the tiles of whole rounds of 256 computed over all of K, only the
# last round's tiles split into K ranges.

def tile_order(tiles_m: int, tiles_n: int, group_m: int = 8):
    """(tile row, tile column) of each tile in the kernels' tile order: groups
    of 8 tile rows, column by column inside a group."""
    order = []
    for g0 in range(0, tiles_m, group_m):
        for tn in range(tiles_n):
            order.extend((g0 + i, tn) for i in range(min(group_m, tiles_m - g0)))
    return order


# (kernel, tile edge, M, K, N): 18 x 16, 17 x 18 and 17 x 17 tiles, ragged
# edges; the last rounds hold 32, 50 and 33 tiles.
TAIL_CASES = [("dma32_64x64_s3", 64, 1100, 777, 1000), ("dma32_128x128_w8_s3", 128, 2100, 200, 2200),
              ("dma32_256x256_w8_s3", 256, 4200, 60, 4300)]


@pytest.mark.parametrize("kname,t,M,K,N", TAIL_CASES, ids=[c[0] for c in TAIL_CASES])
@pytest.mark.parametrize("split", [2, 3, 4])
def test_split_tail_parity_and_structure(kname, t, M, K, N, split):
    """Every output against the oracle; tiles of the whole rounds bit-identical
    to the unsplit plan's, tiles of the last round bit-identical to the plan
    that splits every tile (the same K ranges, summed in the same order)."""
    kid = binding.KERNELS[kname]
    say(f"split tail {kname} {M}x{K}x{N} split {split}")
    A, B = gemm_inputs.draw(M, K, N, "uniform", seed=M + K + N + split)
    C_tail = run(A, B, plan=binding.make_plan(kid, split, True))
    C_ref, S = oracle.gemm(A, B)
    assert_within_bound(C_tail, C_ref, S, f"{kname} tail/{split}")
    C_one = run(A, B, plan=binding.make_plan(kid, 1))
    C_all = run(A, B, plan=binding.make_plan(kid, split))
    order = tile_order(-(-M // t), -(-N // t))
    whole = len(order) // 256 * 256
    assert 0 < whole < len(order)
    for i, (r, c) in enumerate(order):
        rs, cs = slice(r * t, (r + 1) * t), slice(c * t, (c + 1) * t)
        want = C_one if i < whole else C_all
        assert_bits_equal(C_tail[rs, cs], want[rs, cs], f"{kname} tile {i} ({r}, {c})")


@pytest.mark.parametrize("kname,t,M,K,N", TAIL_CASES, ids=[c[0] for c in TAIL_CASES])
def test_split_tail_integers_bit_exact(kname, t, M, K, N):
    say(f"split tail {kname} int {M}x{K}x{N}")
    A, B = gemm_inputs.draw(M, K, N, "int", seed=K + 5)
    C = run(A, B, plan=binding.make_plan(binding.KERNELS[kname], 3, True))
    C_ref = oracle.gemm_i64(A.astype(np.int64), B.astype(np.int64)).astype(np.float32)
    assert_bits_equal(C, C_ref, f"{kname} tail int")


# ---------------------------------------------------------------------------
# The last K steps of a range run as an unrolled copy per remaining count
# (1 .. 2 x stages) in the small-tile copy-fed kernels and as a loop in the
# others: every count, with the last step ragged (K % 4 == 3, so the lanes
# that copied the straddling 16-byte chunks zero its tail) and whole, for
# every copy-fed kernel, whole K and split in two.

DMA_KERNELS = [k for k in binding.KERNELS if k.startswith("dma")]
K_STEP = {k: (32 if k.startswith("dma16_") and k != "dma16_128x128_w4" else 16) for k in DMA_KERNELS}
STEP_COUNTS = [(n, -5) for n in range(1, 17)] + [(n, 0) for n in (6, 7, 8, 10, 11, 15)]


@pytest.mark.parametrize("kname", DMA_KERNELS)
@pytest.mark.parametrize("steps,off", STEP_COUNTS, ids=[f"{n}{'' if o == 0 else 'r'}" for n, o in STEP_COUNTS])
@pytest.mark.parametrize("split", [1, 2])
def test_every_last_step_count(kname, steps, off, split):
    K = K_STEP[kname] * steps + off
    M, N = 70, 90
    say(f"last steps {kname} K {K} ({steps} steps) split {split}")
    A, B = gemm_inputs.draw(M, K, N, "uniform", seed=K * 3 + split)
    C = run(A, B, plan=binding.make_plan(binding.KERNELS[kname], split))
    C_ref, S = oracle.gemm(A, B)
    assert_within_bound(C, C_ref, S, f"{kname} K {K} split {split}")


# A last step of 1 to 4 elements (K = 513 ends one element into its step):
# the small-tile copy-fed kernels read it from global memory into registers
# instead of copying it through the LDS ring; the others stage it as usual.
# Every ring length from 1 to 2 x stages + 1 before it, float and integer
# inputs (the integer sums pin which lane takes which k of the extra step).

RAGGED_STEPS = [2, 3, 4, 5, 7, 8, 13]


@pytest.mark.parametrize("kname", DMA_KERNELS)
@pytest.mark.parametrize("steps", RAGGED_STEPS)
@pytest.mark.parametrize("r", [1, 2, 3, 4])
@pytest.mark.parametrize("split", [1, 2])
def test_short_last_step(kname, steps, r, split):
    K = K_STEP[kname] * (steps - 1) + r
    M, N = 70, 90
    say(f"short last step {kname} K {K} ({steps} steps, {r} in the last) split {split}")
    A, B = gemm_inputs.draw(M, K, N, "uniform", seed=K * 5 + split)
    C = run(A, B, plan=binding.make_plan(binding.KERNELS[kname], split))
    C_ref, S = oracle.gemm(A, B)
    assert_within_bound(C, C_ref, S, f"{kname} K {K} split {split}")


@pytest.mark.parametrize("kname", DMA_KERNELS)
@pytest.mark.parametrize("r", [1, 2, 3, 4])
@pytest.mark.parametrize("split", [1, 2])
def test_short_last_step_integers_bit_exact(kname, r, split):
    K = K_STEP[kname] * 4 + r
    M, N = 130, 97
    say(f"short last step {kname} int K {K} split {split}")
    A, B = gemm_inputs.draw(M, K, N, "int", seed=K + split)
    C = run(A, B, plan=binding.make_plan(binding.KERNELS[kname], split))
    C_ref = oracle.gemm_i64(A.astype(np.int64), B.astype(np.int64)).astype(np.float32)
    assert_bits_equal(C, C_ref, f"{kname} int K {K} split {split}")


PLANNER_TAILS = [((1100, 777, 1000), "dma_mfma32_f32_64x64x16_w4_s3"),
                 ((1792, 1792, 1792), "dma_mfma16_f32_96x96x32_w4_s3")]


@pytest.mark.parametrize("shape,kernel", PLANNER_TAILS, ids=[k for _, k in PLANNER_TAILS])
def test_split_tail_planner(shape, kernel):
    """The planner's split tails: 18 x 16 tiles of 64 x 64 (the last round of
    32 split two ways) and 19 x 19 tiles of 96 x 96 (the last 105 split two
    ways); every output against the oracle, a rerun bit-identical, caller and
    library workspaces bit-identical."""
    M, K, N = shape
    plan = binding.gemm_f32_plan(M, N, K)
    say(f"split tail planner {M}x{K}x{N} plan {plan}")
    assert binding.gemm_kernel_name(plan.kernel) == kernel
    assert plan.split_tail == 1 and plan.split_k > 1
    A, B = gemm_inputs.draw(M, K, N, "uniform", seed=15)
    C1 = run(A, B)
    C_ref, S = oracle.gemm(A, B)
    assert_within_bound(C1, C_ref, S, f"{M}x{K}x{N} split tail")
    assert_bits_equal(run(A, B), C1, "rerun")
    assert_bits_equal(run(A, B, entry="gemm_f32_ex"), C1, "caller workspace")


# ---------------------------------------------------------------------------
# Memory safety, degenerate sizes, API contract.

@pytest.mark.parametrize("kname,kid", KERNELS, ids=[k for k, _ in KERNELS])
@pytest.mark.parametrize("misalign", [0, 1])
def test_guard_bands_untouched(kname, kid, misalign):
    """A, B and C sit inside one NaN-filled buffer with NaN guards around each;
    a read past an operand would turn outputs into NaN, a write past C would
    change a guard. misalign = 1 shifts every operand by one float (the 4-byte
    load path)."""
    t = torch()
    M, K, N, split = 97, 53, 71, 2
    say(f"guard bands {kname} misalign {misalign}")
    A, B = gemm_inputs.draw(M, K, N, "uniform", seed=21)
    g = 256 + misalign
    offA = g
    offB = offA + M * K + g
    offC = offB + K * N + g
    total = offC + M * N + g
    buf = nan_buffer(total)
    buf[offA:offA + M * K] = to_dev(A.ravel())
    buf[offB:offB + K * N] = to_dev(B.ravel())
    plan = binding.make_plan(kid, split)
    need = binding.gemm_f32_plan_workspace_bytes(M, N, K, plan)
    ws = t.empty((max(need // 4, 1),), dtype=t.float32, device="cuda:0")
    base = buf.data_ptr()
    s = t.cuda.current_stream()
    binding.gemm_f32_with_plan(base + 4 * offA, base + 4 * offB, base + 4 * offC, M, N, K, plan,
                               ws, need, s.cuda_stream)
    s.synchronize()
    host = buf.cpu().numpy()
    C = host[offC:offC + M * N].reshape(M, N)
    C_ref, S = oracle.gemm(A, B)
    assert_within_bound(C, C_ref, S, "guarded C")
    guards = np.concatenate([host[:offA], host[offA + M * K:offB], host[offB + K * N:offC],
                             host[offC + M * N:]])
    assert np.isnan(guards).all()
    np.testing.assert_array_equal(host[offA:offA + M * K], A.ravel())
    np.testing.assert_array_equal(host[offB:offB + K * N], B.ravel())


def test_k_zero_writes_positive_zeros():
    t = torch()
    say("K = 0")
    dC = nan_buffer(5 * 7)
    binding.gemm_f32(0, 0, dC, 5, 7, 0, t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    assert (dC.view(t.int32) == 0).all()


def test_empty_outputs_leave_memory_untouched():
    t = torch()
    say("M = 0 / N = 0")
    dC = nan_buffer(16)
    dA = to_dev(np.ones((4, 4), np.float32))
    binding.gemm_f32(dA, dA, dC, 0, 4, 4, 0)
    binding.gemm_f32(dA, dA, dC, 4, 0, 4, 0)
    t.cuda.synchronize()
    assert t.isnan(dC).all()


def test_alias_rejected_before_any_work():
    t = torch()
    say("alias")
    dA = to_dev(np.ones((8, 8), np.float32))
    with pytest.raises(binding.GemmError) as e:
        binding.gemm_f32(dA, dA, dA.data_ptr() + 16, 8, 8, 8, 0)
    assert e.value.status == binding.GEMM_ERR_ALIAS
    t.cuda.synchronize()
    assert (dA == 1).all()


def test_transpose_identity():
    """(AB)^T = B^T A^T: the product of the transposed operands is the
    transpose of the product, within the bound, on the GPU."""
    say("transpose identity")
    A, B = gemm_inputs.draw(300, 129, 170, "uniform", seed=8)
    C = run(A, B)
    Ct = run(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    C_ref, S = oracle.gemm(A, B)
    assert_within_bound(C, C_ref, S, "C")
    assert_within_bound(Ct.T, C_ref, S, "C from transposes")


def test_non_default_stream():
    t = torch()
    say("non-default stream")
    A, B = gemm_inputs.draw(256, 512, 256, "uniform", seed=4)
    stream = t.cuda.Stream()
    C = run(A, B, stream=stream)
    C_ref, S = oracle.gemm(A, B)
    assert_within_bound(C, C_ref, S, "side stream")


def test_calls_do_not_synchronize_the_device():
    """Stream semantics: with a long run of work queued on one stream, calls
    on another stream (an unsplit plan, and a split plan with a caller-owned
    workspace) return while that work is still running, so they did not wait
    for the device; their results are right once their own stream is done."""
    t = torch()
    say("no implicit device synchronisation")
    cases = [(1001, 513, 777), (256, 8192, 256)]
    inputs = []
    for (M, K, N) in cases:
        A, B = gemm_inputs.draw(M, K, N, "uniform", seed=M + N)
        need = binding.gemm_f32_workspace_bytes(M, N, K)
        inputs.append((M, K, N, A, B, to_dev(A), to_dev(B), nan_buffer(M * N), need,
                       t.empty((max(need // 4, 1),), dtype=t.float32, device="cuda:0")))
    x = t.randn(4096, 4096, device="cuda:0")
    busy, side = t.cuda.Stream(), t.cuda.Stream()
    t.cuda.synchronize()
    with t.cuda.stream(busy):
        for _ in range(60):          # tens of milliseconds of matrix products
            y = x @ x
    for (M, K, N, A, B, dA, dB, dC, need, ws) in inputs:
        binding.gemm_f32_ex(dA, dB, dC, M, N, K, ws, need, side.cuda_stream)
    still_running = not busy.query()
    side.synchronize()
    t.cuda.synchronize()
    del y
    assert still_running, "a library call waited for work on another stream"
    for (M, K, N, A, B, dA, dB, dC, need, ws) in inputs:
        C_ref, S = oracle.gemm(A, B)
        assert_within_bound(dC.cpu().numpy().reshape(M, N), C_ref, S, f"{M}x{K}x{N}")


# Sizes at tile and K-step edges (16, 32, 64, 128, 256, 512 and their
# neighbours) and primes, crossed sparsely into (M, K, N) triples.
EDGE_SIZES = [1, 2, 3, 7, 15, 16, 17, 31, 32, 33, 63, 64, 65, 97, 127, 128, 129, 251, 255, 256,
              257, 509, 511, 512, 513]
EDGE_CASES = [(EDGE_SIZES[i % 25], EDGE_SIZES[(7 * i + 3 + i // 25) % 25],
               EDGE_SIZES[(11 * i + 5 + 3 * (i // 25)) % 25]) for i in range(50)]


@pytest.mark.parametrize("M,K,N", EDGE_CASES, ids=[f"{m}x{k}x{n}" for m, k, n in EDGE_CASES])
def test_edge_size_sweep_planner(M, K, N):
    """The planner's plan (gemm_f32) on sizes at every tile and K-step edge:
    each output against the oracle, C pre-filled with NaN."""
    say(f"edge sweep {M}x{K}x{N} plan {binding.gemm_f32_plan(M, N, K)}")
    A, B = gemm_inputs.draw(M, K, N, "uniform", seed=M * 3 + K * 5 + N)
    C = run(A, B)
    C_ref, S = oracle.gemm(A, B)
    assert_within_bound(C, C_ref, S, f"{M}x{K}x{N}")


def test_caller_workspace_matches_library_workspace():
    say("gemm_f32_ex vs gemm_f32 (split-K)")
    M, K, N = 256, 16384, 256
    plan = binding.gemm_f32_plan(M, N, K)
    assert plan.split_k > 1
    A, B = gemm_inputs.draw(M, K, N, "uniform", seed=6)
    C1 = run(A, B)
    C2 = run(A, B, entry="gemm_f32_ex")
    assert_bits_equal(C1, C2, "ex vs library workspace")
    C_ref, S = oracle.gemm(A, B)
    assert_within_bound(C1, C_ref, S, "split-K")


def test_splitk_deterministic_and_matches_unsplit_on_integers():
    say("split-K determinism")
    M, K, N = 300, 4000, 200
    A, B = gemm_inputs.draw(M, K, N, "int", seed=9)
    C_ref = oracle.gemm_i64(A.astype(np.int64), B.astype(np.int64)).astype(np.float32)
    for split in (1, 2, 7, 16):
        plan = binding.make_plan(binding.GEMM_KERNEL_MFMA_128x128, split)
        C = run(A, B, plan=plan)
        assert_bits_equal(C, C_ref, f"split {split}")
    A, B = gemm_inputs.draw(M, K, N, "uniform", seed=9)
    plan = binding.make_plan(binding.GEMM_KERNEL_MFMA_128x128, 7)
    assert_bits_equal(run(A, B, plan=plan), run(A, B, plan=plan), "rerun")


# ---------------------------------------------------------------------------
# Degenerate and large-operand shapes through the planner.

SKINNY = [(1, 4096, 4096), (4096, 4096, 1), (4096, 1, 4096), (1, 131072, 1), (3, 70000, 5)]


@pytest.mark.parametrize("M,K,N", SKINNY, ids=[f"{m}x{k}x{n}" for m, k, n in SKINNY])
def test_skinny_and_outer_products(M, K, N):
    """Vector x matrix, matrix x vector, the K = 1 outer product and long dot
    products, with the planner's plan (split K where it chooses to)."""
    say(f"skinny {M}x{K}x{N} plan {binding.gemm_f32_plan(M, N, K)}")
    A, B = gemm_inputs.draw(M, K, N, "uniform", seed=M + K + N)
    C = run(A, B)
    C_ref, S = oracle.gemm(A, B)
    assert_within_bound(C, C_ref, S, f"{M}x{K}x{N}")


def test_operand_past_2gib_offsets():
    """B of 2 GiB (32768 x 16384): an unsplit copy-fed launch would need copy
    offsets past 2^31 bytes, so such a plan runs the register-staged kernel
    of the same tile (here for the 256 x 256 and the 128 x 64 copy-fed
    kernels); the planner's own plan (split K) and the general form (K passes
    if needed) run copy-fed. Every output against the oracle."""
    t = torch()
    M, K, N = 256, 32768, 16384
    say(f"2 GiB operand {M}x{K}x{N}")
    A, B = gemm_inputs.draw(M, K, N, "normal", seed=99)
    dA, dB = to_dev(A), to_dev(B)
    ref, S = oracle.gemm(A, B)
    del B
    s = t.cuda.current_stream()
    outs = {}
    plans = [(f"fallback {kn}", binding.make_plan(binding.KERNELS[kn], 1))
             for kn in ("dma32_256x256_w8_s3", "dma16_128x64")]
    for name, plan in plans + [("planner", binding.gemm_f32_plan(M, N, K))]:
        say(f"  {name}")
        need = binding.gemm_f32_plan_workspace_bytes(M, N, K, plan)
        ws = t.empty((max(need // 4, 1),), dtype=t.float32, device="cuda:0")
        dC = nan_buffer(M * N)
        binding.gemm_f32_with_plan(dA, dB, dC, M, N, K, plan, ws, need, s.cuda_stream)
        s.synchronize()
        outs[name] = dC.cpu().numpy().reshape(M, N)
        del ws, dC
    dC = nan_buffer(M * N)
    binding.gemm_f32_general(0, 0, M, N, K, 1.0, dA, K, dB, N, 0.0, dC, N, stream=s.cuda_stream)
    s.synchronize()
    outs["general"] = dC.cpu().numpy().reshape(M, N)
    for name, C in outs.items():
        assert_within_bound(C, ref, S, name)


# ---------------------------------------------------------------------------
# IEEE special values in the operands propagate as the definition says: each
# output is a sum of products over all of K and nothing else, so zero-filled
# padding, the K order inside an MFMA and split-K partial sums may neither
# add a NaN nor hide one.

SPECIAL_KERNELS = ["dma32_256x256_w8_s3", "dma32_128x128_w8_s3", "dma32_64x64_s3",
                   "dma32_128x128_w4", "dma16_96x96_s3"]


def _check_special_values(kname, plan, M, K, N, i0, k0, k1, j1, zeros):
    """A NaN at A[i0, k0] makes all of row i0 NaN; a +Inf at B[k1, j1] makes
    C[i, j1] = sign(A[i, k1]) * Inf, and NaN where A[i, k1] = 0 (0 * Inf, at
    the rows in `zeros`); every other output stays finite and within the
    bound of the oracle."""
    A, B = gemm_inputs.draw(M, K, N, "uniform", seed=77)
    A[i0, k0] = np.nan
    B[k1, j1] = np.inf
    A[zeros, k1] = 0.0
    C = run(A, B, plan=plan)
    # What the definition fixes, independently of the oracle.
    want_nan = np.zeros((M, N), dtype=bool)
    want_nan[i0, :] = True
    want_nan[zeros, j1] = True
    assert np.array_equal(np.isnan(C), want_nan), f"{kname}: NaN pattern"
    col = np.delete(np.arange(M), [i0, *zeros])
    assert np.array_equal(C[col, j1], np.where(A[col, k1] > 0, np.inf, -np.inf).astype(np.float32))
    # Everything else against the oracle (which computes the same IEEE sums in FP64).
    C_ref, S = oracle.gemm(A, B)
    assert np.array_equal(np.isnan(C_ref), want_nan)
    fin = np.isfinite(C_ref)
    fin[:, j1] = False
    assert fin.sum() == (M - 1) * (N - 1)
    assert np.isfinite(C[fin]).all()
    err = np.abs(C[fin].astype(np.float64) - C_ref[fin])
    assert (err <= 1e-5 * S[fin] + 1e-6).all(), f"{kname}: worst {err.max()}"


@pytest.mark.parametrize("kname", SPECIAL_KERNELS)
@pytest.mark.parametrize("split", [1, 2])
def test_special_values_propagate(kname, split):
    say(f"special values {kname} split {split}")
    _check_special_values(kname, binding.make_plan(binding.KERNELS[kname], split),
                          300, 700, 260, i0=131, k0=333, k1=650, j1=97, zeros=[5])


def test_special_values_split_tail():
    """The split-tail plan of 1100 x 777 x 1000 on 64 x 64 tiles: tile rows
    0-15 are whole tiles, rows 16-17 (outputs 1024-1099) are split in two
    along K. The NaN row lies in a split tile, the Inf column crosses both
    kinds, and the zero products sit in one of each."""
    say("special values split tail")
    kname = "dma32_64x64_s3"
    _check_special_values(kname, binding.make_plan(binding.KERNELS[kname], 2, True),
                          1100, 777, 1000, i0=1050, k0=100, k1=600, j1=517, zeros=[5, 1060])

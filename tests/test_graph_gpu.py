"""Library calls captured into a HIP graph (through torch.cuda.graph) and
replayed: every replay must equal the eager result bit for bit.

The entry points with caller-owned workspaces (gemm_f32_ex,
gemm_f32_with_plan, gemm_f32_general with a workspace) make no allocation
and no memset, so they can be captured; the split-K cases capture the
partial-product kernel and the reduction (of all tiles, or of the split
last round). Between replays the test runs
eager work of its own and synchronises, and it changes the inputs in place
so a replay that reused stale results would be caught.
"""
import numpy as np
import pytest

import gemm_inputs
from fp32_gemm_07_amd import binding
from gpu_util import say, to_dev, torch

pytestmark = pytest.mark.gpu

# 1792^3: the plan splits only the last round of tiles (its own reduction);
# in the general form (op(A) = A^T) it is the 96 x 96 kernel's transposed
# instantiation, and 4001 x 17 x 3999 the 4-wave 128 x 128 one's.
CASES = [(1001, 513, 777, "plain"), (256, 8192, 256, "plain"), (1792, 1792, 1792, "plain"),
         (300, 513, 260, "general"), (1792, 1792, 1792, "general"), (4001, 17, 3999, "general")]


@pytest.mark.parametrize("M,K,N,form", CASES, ids=[f"{m}x{k}x{n}-{f}" for m, k, n, f in CASES])
def test_graph_replays_match_eager(M, K, N, form):
    t = torch()
    say(f"graph capture {M}x{K}x{N} {form}")
    X, Y = gemm_inputs.draw(M, K, N, "uniform", seed=M + K + N)
    dA, dB = to_dev(X), to_dev(Y)
    dC = t.empty((M, N), dtype=t.float32, device="cuda:0")
    if form == "plain":
        need = binding.gemm_f32_workspace_bytes(M, N, K)
    else:
        need = binding.gemm_f32_general_workspace_bytes(1, 0, M, N, K, M, N)
        dA = to_dev(np.ascontiguousarray(X.T))   # op(A) = A^T, A stored K x M
    ws = t.empty((max(need // 4, 1),), dtype=t.float32, device="cuda:0")

    def call(stream_handle):
        if form == "plain":
            binding.gemm_f32_ex(dA, dB, dC, M, N, K, ws, need, stream_handle)
        else:
            binding.gemm_f32_general(1, 0, M, N, K, 1.5, dA, M, dB, N, 0.0, dC, N, ws, need,
                                     stream_handle)

    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        call(side.cuda_stream)           # warm-up outside capture
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()

    graph = t.cuda.CUDAGraph()
    with t.cuda.graph(graph):
        call(t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()

    for r in range(4):
        # new inputs in place, eager reference, then a replay on the same inputs
        dA.mul_(-1.0 if r % 2 else 0.5)
        dB.add_(0.25)
        call(t.cuda.current_stream().cuda_stream)
        t.cuda.synchronize()
        eager = dC.clone()
        dC.fill_(float("nan"))
        graph.replay()
        t.cuda.synchronize()
        assert t.equal(dC.view(t.int32), eager.view(t.int32)), f"replay {r}"
        assert t.isfinite(dC).all()


def test_library_workspace_refused_under_capture():
    """gemm_f32 with a plan that splits K needs the library's workspace, whose
    bookkeeping has no meaning inside a graph: under capture the call returns
    GEMM_ERR_CAPTURING and enqueues nothing. An unsplit plan needs no
    workspace and captures and replays like the other entry points."""
    t = torch()
    say("graph capture: gemm_f32 split plan refused, unsplit plan captured")
    Ms, Ks, Ns = 256, 8192, 256
    assert binding.gemm_f32_plan(Ms, Ns, Ks).split_k > 1
    X, Y = gemm_inputs.draw(Ms, Ks, Ns, "uniform", seed=7)
    dA, dB = to_dev(X), to_dev(Y)
    dC = t.full((Ms, Ns), float("nan"), dtype=t.float32, device="cuda:0")
    M, K, N = 1001, 513, 777
    assert binding.gemm_f32_plan(M, N, K).split_k == 1
    X2, Y2 = gemm_inputs.draw(M, K, N, "uniform", seed=8)
    dA2, dB2 = to_dev(X2), to_dev(Y2)
    dC2 = t.empty((M, N), dtype=t.float32, device="cuda:0")
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        binding.gemm_f32(dA2, dB2, dC2, M, N, K, side.cuda_stream)   # warm-up outside capture
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()

    statuses = []
    graph = t.cuda.CUDAGraph()
    with t.cuda.graph(graph):
        h = t.cuda.current_stream().cuda_stream
        try:
            binding.gemm_f32(dA, dB, dC, Ms, Ns, Ks, h)
            statuses.append(binding.GEMM_OK)
        except binding.GemmError as e:
            statuses.append(e.status)
        binding.gemm_f32(dA2, dB2, dC2, M, N, K, h)
    t.cuda.synchronize()
    assert statuses == [binding.GEMM_ERR_CAPTURING]
    assert t.isnan(dC).all(), "the refused call wrote C"
    # the refused call works eagerly
    binding.gemm_f32(dA, dB, dC, Ms, Ns, Ks, t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    assert t.isfinite(dC).all()
    for r in range(3):
        dA2.mul_(-0.5)
        binding.gemm_f32(dA2, dB2, dC2, M, N, K, t.cuda.current_stream().cuda_stream)
        t.cuda.synchronize()
        eager = dC2.clone()
        dC2.fill_(float("nan"))
        graph.replay()
        t.cuda.synchronize()
        assert t.equal(dC2.view(t.int32), eager.view(t.int32)), f"replay {r}"

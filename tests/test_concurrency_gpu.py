"""Concurrent use of the library: work enqueued on several streams at once,
and calls from several host threads at once, each with its own buffers and
(for split plans) its own workspace. Every result must equal, bit for bit,
the same call made alone: the plan decides the summation order, not the
timing."""
import threading

import numpy as np
import pytest

import gemm_inputs
from fp32_gemm_07_amd import binding
from gpu_util import nan_buffer, say, to_dev, torch

pytestmark = pytest.mark.gpu

# (M, K, N): unsplit, split K (every tile), split tail, ragged
SHAPES = [(1001, 513, 777), (256, 8192, 256), (1536, 1536, 1536), (300, 2000, 260)]


def _case(M, K, N, seed):
    A, B = gemm_inputs.draw(M, K, N, "uniform", seed=seed)
    need = binding.gemm_f32_workspace_bytes(M, N, K)
    t = torch()
    return {"M": M, "K": K, "N": N, "dA": to_dev(A), "dB": to_dev(B),
            "dC": nan_buffer(M * N), "need": need,
            "ws": t.empty((max(need // 4, 1),), dtype=t.float32, device="cuda:0")}


def _call(c, stream_handle):
    binding.gemm_f32_ex(c["dA"], c["dB"], c["dC"], c["M"], c["N"], c["K"], c["ws"], c["need"],
                        stream_handle)


def _alone(c):
    t = torch()
    dC = c["dC"]
    c["dC"] = nan_buffer(c["M"] * c["N"])
    _call(c, t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    out, c["dC"] = c["dC"].clone(), dC
    return out


def test_streams_interleaved():
    t = torch()
    say("concurrency: four products interleaved on two streams")
    cases = [_case(M, K, N, seed=i) for i, (M, K, N) in enumerate(SHAPES)]
    expected = [_alone(c) for c in cases]
    streams = [t.cuda.Stream(), t.cuda.Stream()]
    for s in streams:
        s.wait_stream(t.cuda.current_stream())
    for rep in range(3):
        for c in cases:
            c["dC"].fill_(float("nan"))
        t.cuda.synchronize()
        for i, c in enumerate(cases):
            _call(c, streams[(i + rep) % 2].cuda_stream)
        t.cuda.synchronize()
        for i, c in enumerate(cases):
            assert t.equal(c["dC"].view(t.int32), expected[i].view(t.int32)), (rep, SHAPES[i])


def test_host_threads():
    t = torch()
    say("concurrency: four host threads, one stream each")
    cases = [_case(M, K, N, seed=10 + i) for i, (M, K, N) in enumerate(SHAPES)]
    expected = [_alone(c) for c in cases]
    errors = []

    def worker(i):
        try:
            s = t.cuda.Stream()
            c = cases[i]
            for _ in range(5):
                with t.cuda.stream(s):
                    c["dC"].fill_(float("nan"))
                _call(c, s.cuda_stream)
                s.synchronize()
                if not t.equal(c["dC"].view(t.int32), expected[i].view(t.int32)):
                    errors.append(f"thread {i} {SHAPES[i]}: result differs")
                    return
        except Exception as e:  # reported below, on the main thread
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors
    assert binding.gemm_last_hip_error() == 0


def test_plans_used_are_the_intended_ones():
    """The shapes above cover an unsplit, a split-every-tile and a split-tail plan."""
    plans = [binding.gemm_f32_plan(M, N, K) for (M, K, N) in SHAPES]
    assert plans[0].split_k == 1
    assert plans[1].split_k > 1 and plans[1].split_tail == 0
    assert plans[2].split_k > 1 and plans[2].split_tail == 1
    assert np.all([p.kernel > 0 for p in plans])

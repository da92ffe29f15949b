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
SHAPES = [(1001, 513, 777), (256, 8192, 256), (1792, 1792, 1792), (300, 2000, 260)]


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


# ---------------------------------------------------------------------------
# The library-owned workspace (gemm_f32): overlapping split-K calls on
# different streams must not share partial-sum buffers, a buffer still in
# use must not be freed when a larger one is needed, and more concurrent
# users than the pool has buffers wait on the device for one.

def _lib_case(M, K, N, seed):
    A, B = gemm_inputs.draw(M, K, N, "uniform", seed=seed)
    return {"M": M, "K": K, "N": N, "dA": to_dev(A), "dB": to_dev(B), "dC": nan_buffer(M * N)}


def _lib_call(c, stream_handle):
    binding.gemm_f32(c["dA"], c["dB"], c["dC"], c["M"], c["N"], c["K"], stream_handle)


def _lib_alone(c):
    t = torch()
    keep = c["dC"]
    c["dC"] = nan_buffer(c["M"] * c["N"])
    _lib_call(c, t.cuda.current_stream().cuda_stream)
    t.cuda.synchronize()
    out, c["dC"] = c["dC"].clone(), keep
    return out


def _busy(stream, n=3):
    """Queue n unsplit 4096^3 products (about a millisecond each) on `stream`,
    so that work enqueued after them stays pending while other streams run.
    The caller keeps the returned buffers alive until it has synchronised."""
    t = torch()
    x = t.full((4096, 4096), 0.5, dtype=t.float32, device="cuda:0")
    y = t.empty_like(x)
    stream.wait_stream(t.cuda.current_stream())
    for _ in range(n):
        binding.gemm_f32(x, x, y, 4096, 4096, 4096, stream.cuda_stream)
    return x, y


def test_library_workspace_overlapping_streams():
    """Split-K calls through gemm_f32 on two streams, each stream held back by
    queued work so that both calls' partial sums are in flight together:
    results bit-identical to each call made alone."""
    t = torch()
    say("library workspace: overlapping split-K calls on two streams")
    shapes = [(256, 16384, 256), (1792, 1792, 1792), (512, 8192, 384)]
    assert all(binding.gemm_f32_plan(M, N, K).split_k > 1 for M, K, N in shapes)
    cases = [_lib_case(M, K, N, seed=30 + i) for i, (M, K, N) in enumerate(shapes)]
    expected = [_lib_alone(c) for c in cases]
    streams = [t.cuda.Stream(), t.cuda.Stream()]
    for rep in range(3):
        for c in cases:
            c["dC"].fill_(float("nan"))
        t.cuda.synchronize()
        keep = [_busy(s) for s in streams]
        for i, c in enumerate(cases):
            _lib_call(c, streams[(i + rep) % 2].cuda_stream)
        t.cuda.synchronize()
        del keep
        for i, c in enumerate(cases):
            assert t.equal(c["dC"].view(t.int32), expected[i].view(t.int32)), (rep, shapes[i])
    assert binding.gemm_last_hip_error() == 0


def test_library_workspace_grows_while_a_buffer_is_in_use():
    """A small split-K call left pending on one stream, then calls needing ever
    larger workspaces on another: the pending call's buffer must survive (it
    is never freed while in use) and every result must match the call made
    alone."""
    t = torch()
    say("library workspace: growth while a buffer is in use")
    small = _lib_case(128, 8192, 128, seed=40)
    bigger = [_lib_case(M, K, N, seed=41 + i)
              for i, (M, K, N) in enumerate([(256, 16384, 256), (512, 32768, 512),
                                             (640, 16384, 640), (800, 32768, 800)])]
    needs = [binding.gemm_f32_workspace_bytes(c["M"], c["N"], c["K"]) for c in [small] + bigger]
    assert all(a < b for a, b in zip(needs, needs[1:])), needs
    exp_small = _lib_alone(small)
    exp_big = [_lib_alone(c) for c in bigger]
    s1, s2 = t.cuda.Stream(), t.cuda.Stream()
    for rep in range(2):
        small["dC"].fill_(float("nan"))
        for c in bigger:
            c["dC"].fill_(float("nan"))
        t.cuda.synchronize()
        keep = _busy(s1, n=5)
        _lib_call(small, s1.cuda_stream)
        for c in bigger:
            _lib_call(c, s2.cuda_stream)
        t.cuda.synchronize()
        del keep
        assert t.equal(small["dC"].view(t.int32), exp_small.view(t.int32)), rep
        for c, e in zip(bigger, exp_big):
            assert t.equal(c["dC"].view(t.int32), e.view(t.int32)), (rep, c["M"])


def test_library_workspace_more_users_than_buffers():
    """Twelve streams, each held back by queued work, each with a split-K call
    of the same shape: more callers at once than the pool keeps buffers
    (eight per device), so some calls wait on the device for a buffer. Every
    result bit-identical to the call made alone."""
    t = torch()
    say("library workspace: twelve concurrent split-K callers")
    M, K, N = 256, 8192, 256
    assert binding.gemm_f32_plan(M, N, K).split_k > 1
    cases = [_lib_case(M, K, N, seed=50 + i) for i in range(12)]
    expected = [_lib_alone(c) for c in cases]
    streams = [t.cuda.Stream() for _ in cases]
    for c in cases:
        c["dC"].fill_(float("nan"))
    t.cuda.synchronize()
    keep = [_busy(s, n=1) for s in streams]
    for c, s in zip(cases, streams):
        _lib_call(c, s.cuda_stream)
    t.cuda.synchronize()
    del keep
    for i, c in enumerate(cases):
        assert t.equal(c["dC"].view(t.int32), expected[i].view(t.int32)), i


def test_library_workspace_host_threads():
    """Four host threads calling gemm_f32 (library workspace) on their own
    streams at once, split and unsplit plans: each result bit-identical to
    the call made alone."""
    t = torch()
    say("library workspace: four host threads")
    cases = [_lib_case(M, K, N, seed=60 + i) for i, (M, K, N) in enumerate(SHAPES)]
    expected = [_lib_alone(c) for c in cases]
    errors = []

    def worker(i):
        try:
            s = t.cuda.Stream()
            c = cases[i]
            for _ in range(5):
                with t.cuda.stream(s):
                    c["dC"].fill_(float("nan"))
                _lib_call(c, s.cuda_stream)
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

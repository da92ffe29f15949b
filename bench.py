"""Bench: FP32 GEMM throughput (2MNK/s) on one MI355X, through the C ABI.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
    python bench.py --sweep [MxKxN ...]      plan sweep (every kernel x split)
    python bench.py --ladder                 the walkthrough's v0..v4 rungs and the MFMA kernels
    python bench.py --orders [MxKxN ...]     the general form in every transpose case
    python bench.py --copy-probe-mib 256     a plain copy of known size (counter calibration)

A step is one C = A x B call of the planner's plan (every kernel it launches,
split-K reduce included) on inputs already resident in HBM. First an untimed
clock-settle pass: the same step back to back for --settle-ms of wall time
(the chip raises its shader clock over the first ~30 ms of sustained load,
and launches timed inside that ramp run up to 25 % slower); then W untimed
warm-up steps; then K timed steps (default: about 20 ms of work at the
settle pass's rate, at least 100) back to back between two device
synchronisations (host wall clock: `value`) and between two HIP events on the
stream they are launched on (device time / K: the mean launch duration of the
roofline); then a short pass of up to 20 launches, each between its own event
pair, for the spread of single launches (context only). One JSON line on
stdout, with the driver's top shader-clock level (`device.max_sclk_mhz`) and
the lowest mean clock the achieved rate allows (`device.sclk_mhz_at_least`).

The CPU baseline is the oracle (plain FP64 triple loop) run on the host's
cores on a bounded slab of rows of the same product (all of C at the five
standing workloads), scaled to TFLOP/s; the same rows of the GPU result are
compared with it.

The sweep, ladder and orders modes time many calls (median or mean of HIP
event pairs around single launches, inputs resident, after a settle pass)
and print one JSON line per case; they check nothing (the tests do).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import gemm_inputs  # noqa: E402
from fp32_gemm_07_amd import binding, roofline  # noqa: E402

METRIC = "FP32 GEMM TFLOPS (2MNK/s) and % of MI355X FP32 peak, 1 GPU"
DEFAULT_WORKLOAD = "square_4096"
# Timed work the default step count aims at (the fixed cost of the two
# synchronisations around the timed region, ~25 us, then stays below 0.2 %).
DEFAULT_TIMED_MS = 20.0

# HBM traffic per launch from two rocprofv3 --pmc runs of this bench
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), keyed by (workload, kernel
# name), with the SHA-256 of the kernel source they were taken on. The raw
# counters are scaled by what they read for a plain copy of known size
# (bench.py --copy-probe-mib 256): FETCH_SIZE x 2.0, WRITE_SIZE x 1.0.
FETCH_FACTOR = 2.0
WRITE_FACTOR = 1.0
_SHA = "f30ed178372ee15e0bab5a0fa975ecf47220d85ed8ed3c4b84d83533c076b668"
MEASURED_TRAFFIC = {
    ("square_4096", "dma_mfma32_f32_256x256x16_w8_s3"): {
        "fetch_kib": 196745.84375, "write_kib": 65536.0, "kernel_source_sha256": _SHA},
    ("longk_512x131072x512", "dma_mfma32_f32_128x128x16_w8_s3"): {
        "fetch_kib": 262244.0, "write_kib": 16384.0, "kernel_source_sha256": _SHA},
    ("regular_1024x512x1024", "dma_mfma32_f32_64x64x16_w4_s3"): {
        "fetch_kib": 6243.0, "write_kib": 4096.0, "kernel_source_sha256": _SHA},
    ("irregular_1001x513x777", "dma_mfma32_f32_64x64x16_w4_s3"): {
        "fetch_kib": 6306.875, "write_kib": 3147.59375, "kernel_source_sha256": _SHA},
    ("small_128x96x112", "dma_mfma32_f32_64x64x16_w4_s3"): {
        "fetch_kib": 147.0, "write_kib": 56.0, "kernel_source_sha256": _SHA},
}
KERNEL_SOURCE = os.path.join(ROOT, "fp32_gemm_07_amd", "csrc", "gemm_kernels.hpp")


def kernel_source_sha() -> str:
    import hashlib
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload: str, kernel: str):
    """Scaled HBM bytes per launch, or None if not measured on this kernel source."""
    m = MEASURED_TRAFFIC.get((workload, kernel))
    if not m or m["kernel_source_sha256"] != kernel_source_sha():
        return None
    return int(round(FETCH_FACTOR * m["fetch_kib"] * 1024 + WRITE_FACTOR * m["write_kib"] * 1024))


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None,
                   help="timed steps (default: about 20 ms of timed work at the settle pass's rate, "
                        "at least 100)")
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--settle-ms", type=float, default=200.0,
                   help="untimed back-to-back steps for at least this much wall time before the "
                        "warm-up steps (the shader clock's ramp under sustained load)")
    p.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=[w.name for w in gemm_inputs.WORKLOADS])
    p.add_argument("--shape", metavar="MxKxN",
                   help="instead of a standing workload, this shape (uniform [-1, 1) inputs, seed 0), "
                        "for profiles of plans the five workloads do not use (e.g. a split tail)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="bound on the wall time of the oracle's CPU-baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--kernel", default="auto", choices=["auto", *binding.KERNELS],
                   help="time this kernel instead of the planner's choice")
    p.add_argument("--split", type=int, default=1, help="split-K ranges for --kernel")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="instead of the bench, run a plain device-to-device copy of this many MiB "
                        "--steps times (calibrates the HBM byte counters against a known size)")
    p.add_argument("--sweep", nargs="*", metavar="MxKxN",
                   help="plan sweep over these shapes (default: a standing list)")
    p.add_argument("--ladder", action="store_true",
                   help="the optimisation ladder on the walkthrough's two shapes")
    p.add_argument("--orders", nargs="*", metavar="MxKxN",
                   help="the general form in every transpose case over these shapes")
    return p.parse_args(argv)


def settle(step, sync, ms: float):
    """Run step() back to back for at least `ms` milliseconds of wall time
    (untimed), in doubling batches each ended by sync(). Returns (wall ms,
    steps)."""
    t0 = time.perf_counter()
    n, batch = 0, 1
    while True:
        for _ in range(batch):
            step()
        n += batch
        sync()
        elapsed = (time.perf_counter() - t0) * 1e3
        if elapsed >= ms:
            return elapsed, n
        batch = min(2 * batch, 4096)


def copy_probe(mib: int, steps: int) -> int:
    """A plain copy of known size: reads and writes mib MiB per launch."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read_per_launch": 4 * n, "bytes_written_per_launch": 4 * n,
                      "launches": steps, "ok": bool(torch.equal(dst, src))}), flush=True)
    return 0


def sclk_table(props):
    """Path of this GPU's shader-clock DPM table in sysfs (amdgpu), or None.
    Its lines are the clock levels ("1: 2400Mhz") and, marked with '*', the
    current clock (a level, or "S: <MHz>" between levels)."""
    import glob
    try:
        dev = f"{props.pci_domain_id:04x}:{props.pci_bus_id:02x}:{props.pci_device_id:02x}.0"
        path = f"/sys/bus/pci/devices/{dev}/pp_dpm_sclk"
        if os.path.exists(path):
            return path
    except AttributeError:
        pass
    paths = glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")
    return paths[0] if len(paths) == 1 else None


def read_sclk(path):
    """(current MHz, highest level MHz) from the DPM table, None where absent."""
    cur, top = None, None
    try:
        with open(path) as f:
            for line in f:
                head, _, rest = line.partition(":")
                mhz = float(rest.strip().split("Mhz")[0].split("MHz")[0])
                if "*" in rest:
                    cur = mhz
                if head.strip().isdigit():
                    top = mhz if top is None else max(top, mhz)
    except (OSError, ValueError):
        pass
    return cur, top


def cpu_sample_rows(M: int, rows_per_s: float, target_s: float) -> int:
    """Rows of C the CPU baseline computes: all of them when the oracle finishes
    C within target_s at the calibrated rate, else as many as fit (never
    fewer than one)."""
    return int(max(1, min(M, rows_per_s * target_s)))


def cpu_baseline(A, B, C_gpu, target_s: float):
    """Time the oracle on a slab of rows of the same product (bounded to about
    target_s seconds of host time); compare those rows with the GPU result."""
    import oracle
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build(force=True)
    M, K = A.shape
    N = B.shape[1]
    threads = oracle.num_threads()
    # calibrate on a few rows, then size the slab
    r0 = min(M, 4 * max(1, threads))
    t0 = time.perf_counter()
    oracle.gemm(A[:r0], B)
    dt0 = max(time.perf_counter() - t0, 1e-6)
    rows = max(r0, cpu_sample_rows(M, r0 / dt0, target_s))
    t0 = time.perf_counter()
    C_ref, S = oracle.gemm(A[:rows], B)
    dt = time.perf_counter() - t0
    flops = roofline.gemm_flops(rows, N, K)
    err = np.abs(C_gpu[:rows].astype(np.float64) - C_ref)
    ratio = float(np.max(err / (1e-5 * S + 1e-6))) if err.size else 0.0
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"rows 0..{rows - 1} of C ({rows} x {N} outputs{', all of C' if rows == M else ''}, "
                  f"full K = {K}), {flops / 1e9:.2f} GFLOP in {dt:.2f} s, FP64 accumulation",
        "seconds": dt,
        "sample_parity_worst_ratio": ratio,
    }


# ---------------------------------------------------------------------------
# Timing modes: sweep, ladder, orders.

SWEEP_SHAPES = [
    "128x96x112", "512x512x512", "1024x512x1024", "1001x513x777", "1024x1024x1024",
    "2048x2048x2048", "1024x4096x1024", "2048x512x2048", "3000x3000x3000", "4096x1024x4096",
    "8192x1024x8192", "256x8192x256", "512x131072x512", "4096x4096x4096", "6144x6144x6144",
    "8192x8192x8192",
]
SWEEP_KERNELS = ["dma32_256x256_w8_s3", "dma32_256x256_w8", "dma32_128x128_w4",
                 "dma32_128x128_w8_s3", "dma32_128x128_w8", "dma16_128x128_w4", "dma16_96x96_s3",
                 "dma32_64x64_s3", "dma32_64x64", "dma16_64x64", "dma16_128x64", "mfma16_64x64",
                 "mfma32_128x128", "mfma32_64x64", "valu_64x64"]
SWEEP_SPLITS = (1, 2, 4, 8, 16, 32, 64)
SWEEP_MAX_WORKSPACE = 2 << 30
# copy-fed kernels that take a split tail, by tile edge
TAIL_KERNELS = {"dma32_256x256_w8_s3": 256, "dma32_128x128_w8_s3": 128, "dma16_96x96_s3": 96,
                "dma32_64x64_s3": 64}

LADDER_SHAPES = ["1024x512x1024", "1001x513x777"]
# The walkthrough's rungs v0..v4, then the matrix-core kernels.
LADDER = [("v0 naive, lanes along rows", "ladder_v0"), ("v1 naive, lanes along columns", "ladder_v1"),
          ("v2 LDS tiles 16x16", "ladder_v2"), ("v3 LDS, 4 outputs per lane", "ladder_v3"),
          ("v4 LDS, 4x4 outputs per lane", "valu_64x64"),
          ("MFMA 32x32x2, register-staged 64x64", "mfma32_64x64"),
          ("MFMA 32x32x2, copy-fed 64x64", "dma32_64x64_s3")]

ORDER_SHAPES = ["4096x4096x4096", "1024x512x1024", "1001x513x777", "2048x1024x2048",
                "512x131072x512"]


def parse_shape(s: str):
    M, K, N = (int(v) for v in s.lower().split("x"))
    return M, K, N


def plan_label(plan) -> str:
    return (f"{binding.gemm_kernel_name(plan.kernel)}/S{plan.split_k}"
            + ("t" if plan.split_tail else ""))


class Timer:
    """HIP event pairs around single launches on torch's current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.stream = torch.cuda.current_stream()

    def times_us(self, call, reps: int, warm: int = 3):
        t = self.torch
        for _ in range(warm):
            call()
        t.cuda.synchronize()
        ev = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for e0, e1 in ev:
            e0.record(self.stream)
            call()
            e1.record(self.stream)
        t.cuda.synchronize()
        return np.array([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev])

    def median_us(self, call, reps: int) -> float:
        return float(np.median(self.times_us(call, reps)))


def reps_for(flop: float) -> int:
    """Launches to time: about 0.15 s of work, between 5 and 200."""
    return max(5, min(200, int(0.15 / max(flop / 120e12, 1e-6))))


def settle_gpu(torch, ms: float) -> dict:
    """The settle pass of the timing modes: a 4096^3 product of the library,
    back to back, for `ms` of wall time."""
    x = torch.rand((4096, 4096), device="cuda:0")
    y = torch.empty_like(x)
    h = torch.cuda.current_stream().cuda_stream
    plan = binding.gemm_f32_plan(4096, 4096, 4096)
    el, n = settle(lambda: binding.gemm_f32_with_plan(x, x, y, 4096, 4096, 4096, plan, None, 0, h),
                   torch.cuda.synchronize, ms)
    return {"ms": round(el, 1), "steps": n, "product": "4096x4096x4096"}


def vendor_matmul(torch, a, b, out):
    torch.backends.cuda.matmul.allow_tf32 = False
    return lambda: torch.matmul(a, b, out=out)


def run_sweep(torch, shapes, settle_ms: float) -> int:
    """Every kernel x split (x split tail) of each shape, the planner's plan and
    torch.matmul in FP32 (the vendor library, context only): medians of event
    pairs around back-to-back launches. One JSON line per shape."""
    timer = Timer(torch)
    h = timer.stream.cuda_stream
    gen = torch.Generator(device="cuda").manual_seed(0)
    print(json.dumps({"mode": "sweep", "settle": settle_gpu(torch, settle_ms)}), flush=True)
    for shape in shapes:
        M, K, N = parse_shape(shape)
        dA = torch.rand((M, K), device="cuda", generator=gen) * 2 - 1
        dB = torch.rand((K, N), device="cuda", generator=gen) * 2 - 1
        dC = torch.empty((M, N), device="cuda")
        flop = roofline.gemm_flops(M, N, K)
        reps = reps_for(flop)

        def plan_call(plan):
            need = binding.gemm_f32_plan_workspace_bytes(M, N, K, plan)
            ws = torch.empty(max(need // 4, 1), device="cuda")
            return lambda: binding.gemm_f32_with_plan(dA, dB, dC, M, N, K, plan, ws, need, h)

        res = []
        for kn in SWEEP_KERNELS:
            for sp in SWEEP_SPLITS:
                if sp > 1 and K // sp < 256:
                    continue
                tails = [False]
                if sp > 1 and kn in TAIL_KERNELS:
                    t = TAIL_KERNELS[kn]
                    tiles = -(-M // t) * -(-N // t)
                    if tiles > 256 and tiles % 256:
                        tails.append(True)
                for tail in tails:
                    plan = binding.make_plan(binding.KERNELS[kn], sp, tail)
                    if binding.gemm_f32_plan_workspace_bytes(M, N, K, plan) > SWEEP_MAX_WORKSPACE:
                        continue
                    res.append((timer.median_us(plan_call(plan), reps),
                                f"{kn}/S{sp}" + ("t" if tail else "")))
        auto = binding.gemm_f32_plan(M, N, K)
        t_auto = timer.median_us(plan_call(auto), reps)
        t_vendor = timer.median_us(vendor_matmul(torch, dA, dB, dC), reps)
        res.sort()
        print(json.dumps({
            "mode": "sweep", "shape": f"{M}x{K}x{N}", "M": M, "K": K, "N": N,
            "planner": {"plan": plan_label(auto), "us": round(t_auto, 2),
                        "tflops": round(flop / t_auto / 1e6, 2)},
            "vendor_torch_matmul": {"us": round(t_vendor, 2), "tflops": round(flop / t_vendor / 1e6, 2)},
            "fastest": [{"plan": name, "us": round(us, 2)} for us, name in res[:4]],
            "all": {name: round(us, 2) for us, name in res},
            "plans_timed": len(res), "reps": reps, "timing": "median of event pairs"}), flush=True)
    return 0


def run_ladder(torch, settle_ms: float) -> int:
    """Each rung of the ladder on the walkthrough's two shapes: the mean of 50
    launches after 3 warm-ups, as in its tables. One JSON line per rung."""
    timer = Timer(torch)
    h = timer.stream.cuda_stream
    gen = torch.Generator(device="cuda").manual_seed(0)
    print(json.dumps({"mode": "ladder", "settle": settle_gpu(torch, settle_ms)}), flush=True)
    for shape in LADDER_SHAPES:
        M, K, N = parse_shape(shape)
        dA = torch.rand((M, K), device="cuda", generator=gen) * 2 - 1
        dB = torch.rand((K, N), device="cuda", generator=gen) * 2 - 1
        dC = torch.empty((M, N), device="cuda")
        flop = roofline.gemm_flops(M, N, K)
        t_vendor = float(np.mean(timer.times_us(vendor_matmul(torch, dA, dB, dC), 50)))
        for label, kn in LADDER + [("torch.matmul FP32 (vendor library)", None)]:
            if kn is None:
                us, name = t_vendor, "torch.matmul"
            else:
                plan = binding.make_plan(binding.KERNELS[kn], 1)
                us = float(np.mean(timer.times_us(
                    lambda: binding.gemm_f32_with_plan(dA, dB, dC, M, N, K, plan, None, 0, h), 50)))
                name = binding.gemm_kernel_name(plan.kernel)
            print(json.dumps({"mode": "ladder", "shape": shape, "rung": label, "kernel": name,
                              "us_mean_of_50": round(us, 2), "gflops": round(flop / us / 1e3, 1),
                              "vendor_us_over_us": round(t_vendor / us, 4)}), flush=True)
    return 0


def run_orders(torch, shapes, settle_ms: float) -> int:
    """gemm_f32_general in the four transpose cases, with alpha = 1, beta = 0
    and alpha = 2, beta = 0.5, next to torch.matmul on the same (transposed)
    storage: medians of event pairs. One JSON line per shape and case."""
    timer = Timer(torch)
    h = timer.stream.cuda_stream
    gen = torch.Generator(device="cuda").manual_seed(0)
    print(json.dumps({"mode": "orders", "settle": settle_gpu(torch, settle_ms)}), flush=True)
    for shape in shapes:
        M, K, N = parse_shape(shape)
        flop = roofline.gemm_flops(M, N, K)
        reps = reps_for(flop)
        C = torch.rand((M, N), device="cuda", generator=gen)
        for ta, tb in ((0, 0), (1, 0), (0, 1), (1, 1)):
            A = torch.rand((K, M) if ta else (M, K), device="cuda", generator=gen)
            B = torch.rand((N, K) if tb else (K, N), device="cuda", generator=gen)
            lda, ldb = A.shape[1], B.shape[1]
            need = binding.gemm_f32_general_workspace_bytes(ta, tb, M, N, K, lda, ldb)
            ws = torch.empty(max(need // 4, 1), device="cuda")
            res = {}
            for alpha, beta in ((1.0, 0.0), (2.0, 0.5)):
                res[(alpha, beta)] = timer.median_us(
                    lambda: binding.gemm_f32_general(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta,
                                                     C, N, ws, need, h), reps)
            t_v = timer.median_us(vendor_matmul(torch, A.t() if ta else A, B.t() if tb else B, C),
                                  reps)
            print(json.dumps({
                "mode": "orders", "shape": shape, "case": "NT"[ta] + "NT"[tb],
                "alpha1_beta0": {"us": round(res[(1.0, 0.0)], 2),
                                 "tflops": round(flop / res[(1.0, 0.0)] / 1e6, 2)},
                "alpha2_beta0.5": {"us": round(res[(2.0, 0.5)], 2),
                                   "tflops": round(flop / res[(2.0, 0.5)] / 1e6, 2)},
                "vendor_torch_matmul": {"us": round(t_v, 2), "tflops": round(flop / t_v / 1e6, 2)},
                "reps": reps, "timing": "median of event pairs"}), flush=True)
    return 0


# ---------------------------------------------------------------------------

def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); the library "
              "has no multi-GPU path (sharding is a design note, not code).", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if args.copy_probe_mib:
        return copy_probe(args.copy_probe_mib, args.steps or 100)
    if args.sweep is not None:
        return run_sweep(torch, args.sweep or SWEEP_SHAPES, args.settle_ms)
    if args.ladder:
        return run_ladder(torch, args.settle_ms)
    if args.orders is not None:
        return run_orders(torch, args.orders or ORDER_SHAPES, args.settle_ms)
    if args.shape:
        Ms, Ks, Ns = parse_shape(args.shape)
        w = gemm_inputs.Workload(f"shape_{Ms}x{Ks}x{Ns}", Ms, Ks, Ns, "uniform", 0)
    else:
        w = gemm_inputs.BY_NAME[args.workload]
    M, N, K = w.M, w.N, w.K
    if args.kernel == "auto":
        plan = binding.gemm_f32_plan(M, N, K)
    else:
        plan = binding.make_plan(binding.KERNELS[args.kernel], args.split)
    kname = binding.gemm_kernel_name(plan.kernel)
    ws_bytes = binding.gemm_f32_plan_workspace_bytes(M, N, K, plan)

    A, B = gemm_inputs.draw_workload(w)
    dev = torch.device("cuda:0")
    dA = torch.from_numpy(A).to(dev)
    dB = torch.from_numpy(B).to(dev)
    dC = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty((max(ws_bytes // 4, 1),), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    h = stream.cuda_stream

    def step():
        binding.gemm_f32_with_plan(dA, dB, dC, M, N, K, plan, ws, ws_bytes, h)

    settle_ms, settle_steps = settle(step, torch.cuda.synchronize, args.settle_ms)
    if args.steps is None:   # the fixed cost around the timed region stays below ~0.2 %
        per_step_ms = settle_ms / settle_steps if settle_steps else 1.0
        args.steps = max(100, int(round(DEFAULT_TIMED_MS / per_step_ms)))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K back-to-back steps, one event pair on the launch stream
    # around all of them (an event record between steps would add its own
    # packet to every step), host wall clock around the same region.
    region = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region[0].record(stream)
    for _ in range(args.steps):
        step()
    region[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_launch_ms = region[0].elapsed_time(region[1]) / args.steps

    # Spread of single launches (context only): a short pass with an event
    # pair around each launch.
    launch_ms = Timer(torch).times_us(step, min(args.steps, 20), warm=0) / 1e3

    props = torch.cuda.get_device_properties(0)
    sclk_path = sclk_table(props)
    max_mhz = read_sclk(sclk_path)[1] if sclk_path else None

    flops = roofline.gemm_flops(M, N, K)
    value = flops * args.steps / wall / 1e12
    achieved = flops / (mean_launch_ms * 1e-3) / 1e12
    peak = roofline.PEAK_FP32_MFMA_TFLOPS

    C = dC.cpu().numpy()
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "M": M, "N": N, "K": K, "dist": w.dist, "seed": w.seed,
            "plan": {"kernel": kname,
                     "split_k": plan.split_k if args.kernel == "auto" else args.split,
                     "split_tail": bool(plan.split_tail)},
            "parallelism": "1 GPU",
        },
        "pct_of_fp32_peak": round(100 * value / peak, 2),
        # untimed, before the warm-up steps: the same step back to back
        "settle": {"ms": round(settle_ms, 1), "steps": settle_steps},
        "launch_ms": {"mean": round(float(mean_launch_ms), 4),
                      "single_launch_median": round(float(np.median(launch_ms)), 4),
                      "single_launch_min": round(float(launch_ms.min()), 4)},
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(w.name, kname),
            "algorithmic_flop_per_launch": flops,
            "compulsory_bytes_per_launch": roofline.compulsory_bytes(M, N, K),
            "kernel": kname,
        },
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", ""), "max_sclk_mhz": max_mhz,
                   # The FP32 matrix cores retire at most 256 FLOP per clock
                   # per CU: the mean shader clock of the timed launches was at
                   # least this.
                   "sclk_mhz_at_least": round(achieved * 1e6 / (props.multi_processor_count * 256), 1)},
        "output_finite": bool(np.isfinite(C).all()),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(A, B, C, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Bench: FP32 GEMM throughput (2MNK/s) on one MI355X, through the C ABI.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one C = A x B call of the planner's plan (every kernel it launches,
split-K reduce included) on inputs already resident in HBM. W untimed steps,
then K timed steps back to back between two device synchronisations (host
wall clock: `value`) and between two HIP events on the stream they are
launched on (device time / K: the mean launch duration of the roofline);
then a short pass of up to 20 launches, each between its own event pair,
for the spread of single launches (context only). One JSON line on stdout,
with the driver's top shader-clock level (`device.max_sclk_mhz`) and the
lowest mean clock the achieved rate allows (`device.sclk_mhz_at_least`).

The CPU baseline is the oracle (plain FP64 triple loop) run on the host's
cores on a bounded slab of rows of the same product, scaled to TFLOP/s; the
same rows of the GPU result are compared with it.
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

# HBM traffic per launch from two rocprofv3 --pmc runs of this bench
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), keyed by (workload, kernel
# name), with the SHA-256 of the kernel source they were taken on. The raw
# counters are scaled by what they read for a plain copy of known size
# (bench.py --copy-probe-mib 256): FETCH_SIZE x 2.0, WRITE_SIZE x 1.0.
FETCH_FACTOR = 2.0
WRITE_FACTOR = 1.0
_SHA = "cc0fc5e33b026f184fd1b5df25d7afe94848e17d5ee9c4c3ad9bff1dc66a59cf"
MEASURED_TRAFFIC = {
    ("square_4096", "dma_mfma32_f32_256x256x16_w8_s3"): {
        "fetch_kib": 196726.0, "write_kib": 65536.0, "kernel_source_sha256": _SHA},
    ("longk_512x131072x512", "dma_mfma32_f32_128x128x16_w8_s3"): {
        "fetch_kib": 262244.53125, "write_kib": 16384.0, "kernel_source_sha256": _SHA},
    ("regular_1024x512x1024", "dma_mfma32_f32_64x64x16_w4_s3"): {
        "fetch_kib": 6224.0, "write_kib": 4096.0, "kernel_source_sha256": _SHA},
    ("irregular_1001x513x777", "dma_mfma32_f32_64x64x16_w4_s3"): {
        "fetch_kib": 6290.125, "write_kib": 3147.59375, "kernel_source_sha256": _SHA},
    ("small_128x96x112", "dma_mfma32_f32_64x64x16_w4_s3"): {
        "fetch_kib": 140.375, "write_kib": 56.0, "kernel_source_sha256": _SHA},
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
    p.add_argument("--steps", type=int, default=100)
    # The chip ramps its clock over the first ~30 ms of sustained MFMA load
    # (per-dispatch kernel traces: 1.1-1.2 ms at first, steady after ~30
    # dispatches at 4096^3); 50 untimed steps put the timed ones past it.
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=[w.name for w in gemm_inputs.WORKLOADS])
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target wall time of the oracle's CPU-baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--kernel", default="auto", choices=["auto", *binding.KERNELS],
                   help="time this kernel instead of the planner's choice")
    p.add_argument("--split", type=int, default=1, help="split-K ranges for --kernel")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="instead of the bench, run a plain device-to-device copy of this many MiB "
                        "--steps times (calibrates the HBM byte counters against a known size)")
    return p.parse_args(argv)


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
    rows = int(min(M, max(r0, r0 * target_s / dt0)))
    rows = max(threads, (rows // threads) * threads) if rows >= threads else rows
    rows = min(rows, M)
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
        "sample": f"rows 0..{rows - 1} of C ({rows} x {N} outputs, full K = {K}), "
                  f"{flops / 1e9:.2f} GFLOP in {dt:.2f} s, FP64 accumulation",
        "seconds": dt,
        "sample_parity_worst_ratio": ratio,
    }


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
        return copy_probe(args.copy_probe_mib, args.steps)
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
    n_each = min(args.steps, 20)
    each = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(n_each)]
    for e0, e1 in each:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    launch_ms = np.array([e0.elapsed_time(e1) for e0, e1 in each])

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

"""Time every copy-fed and register-staged plan over a list of shapes.

    python -m fp32_gemm_07_amd.sweep [MxKxN ...]
    python -m fp32_gemm_07_amd.sweep --ladder
    python -m fp32_gemm_07_amd.sweep --orders [MxKxN ...]

For each shape: the planner's choice, torch.matmul in FP32 (the vendor
library, for context), and the four fastest (kernel, split) plans, each the
median of HIP-event timings of back-to-back launches on inputs resident on
the GPU (uniform [-1, 1) values; timing only, nothing is checked). This is
the measurement the planner's cost model is fitted to. "S4" splits every
tile into 4 K ranges; "S4t" only the tiles of the last, partial round of
256 (the planner's kernels, shapes with such a round).

--ladder times the optimisation ladder of the yekq.top LeetGPU walkthrough
(v0 .. v4, then the matrix-core kernels) on its two shapes, 1024 x 512 x 1024
and 1001 x 513 x 777, with the mean of 50 launches as in its tables.

--orders times gemm_f32_general for the four transpose cases, with
alpha = 1, beta = 0 and with alpha = 2, beta = 0.5, next to torch.matmul on
the same (transposed) storage.
"""
from __future__ import annotations

import sys

from . import binding, roofline

DEFAULT_SHAPES = [
    "128x96x112", "512x512x512", "1024x512x1024", "1001x513x777", "1024x1024x1024",
    "2048x2048x2048", "1024x4096x1024", "2048x512x2048", "3000x3000x3000", "4096x1024x4096",
    "8192x1024x8192", "256x8192x256", "512x131072x512", "4096x4096x4096", "6144x6144x6144",
    "8192x8192x8192",
]
KERNELS = ["dma32_256x256_w8_s3", "dma32_256x256_w8", "dma32_128x128_w4", "dma32_128x128_w8_s3",
           "dma32_128x128_w8",
           "dma16_128x128_w4",
           "dma32_64x64_s3", "dma32_64x64", "dma16_64x64", "dma16_128x64", "mfma16_64x64", "mfma32_128x128",
           "mfma32_64x64", "valu_64x64"]
SPLITS = (1, 2, 4, 8, 16, 32, 64)
MAX_WORKSPACE = 2 << 30
TAIL_KERNELS = {"dma32_256x256_w8_s3": 256, "dma32_128x128_w8_s3": 128, "dma32_64x64_s3": 64}


def plan_label(plan) -> str:
    return f"S{plan.split_k}" + ("t" if plan.split_tail else "")


LADDER_SHAPES = ["1024x512x1024", "1001x513x777"]
# The walkthrough's rungs v0..v4, then the matrix-core kernels.
LADDER = [("v0 naive, lanes along rows", "ladder_v0"), ("v1 naive, lanes along columns", "ladder_v1"),
          ("v2 LDS tiles 16x16", "ladder_v2"), ("v3 LDS, 4 outputs per lane", "ladder_v3"),
          ("v4 LDS, 4x4 outputs per lane", "valu_64x64"),
          ("MFMA 32x32x2, register-staged 64x64", "mfma32_64x64"),
          ("MFMA 32x32x2, copy-fed 64x64", "dma32_64x64_s3")]


def ladder(np, torch) -> int:
    """Each rung of the ladder on the pages' two shapes, as in their tables."""
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device="cuda").manual_seed(0)
    # ~0.1 s of matrix-core load first: the clock ramps up over the first
    # tens of milliseconds of sustained load.
    x = torch.rand((2048, 2048), device="cuda", generator=gen)
    for _ in range(100):
        torch.matmul(x, x)
    torch.cuda.synchronize()
    for shape in LADDER_SHAPES:
        M, K, N = (int(x) for x in shape.split("x"))
        dA = torch.rand((M, K), device="cuda", generator=gen) * 2 - 1
        dB = torch.rand((K, N), device="cuda", generator=gen) * 2 - 1
        dC = torch.empty((M, N), device="cuda")
        flop = roofline.gemm_flops(M, N, K)

        def timeit(call, reps=50):
            for _ in range(3):
                call()
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(reps)]
            for e0, e1 in ev:
                e0.record(stream)
                call()
                e1.record(stream)
            torch.cuda.synchronize()
            return float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3

        torch.backends.cuda.matmul.allow_tf32 = False
        t_vendor = timeit(lambda: torch.matmul(dA, dB, out=dC))
        print(f"{shape} (M x K x N): mean of 50 launches after 3 warm-ups", flush=True)
        print(f"  {'rung':40s} {'kernel':36s} {'us':>9s} {'GFLOP/s':>10s} {'vs vendor':>9s}")
        for label, kn in LADDER:
            plan = binding.make_plan(binding.KERNELS[kn], 1)
            us = timeit(lambda: binding.gemm_f32_with_plan(dA, dB, dC, M, N, K, plan, None, 0,
                                                           stream.cuda_stream))
            print(f"  {label:40s} {binding.gemm_kernel_name(plan.kernel):36s} {us:9.2f} "
                  f"{flop / us / 1e3:10.1f} {t_vendor / us:9.1%}", flush=True)
        print(f"  {'torch.matmul FP32 (vendor library)':40s} {'':36s} {t_vendor:9.2f} "
              f"{flop / t_vendor / 1e3:10.1f} {1:9.1%}", flush=True)
    return 0


ORDER_SHAPES = ["4096x4096x4096", "1024x512x1024", "1001x513x777", "2048x1024x2048",
                "512x131072x512"]


def orders(np, torch, shapes) -> int:
    """gemm_f32_general for every transpose case, and with alpha, beta, next to
    torch.matmul on the same storage (transposed views)."""
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device="cuda").manual_seed(0)
    x = torch.rand((2048, 2048), device="cuda", generator=gen)
    for _ in range(100):
        torch.matmul(x, x)
    torch.cuda.synchronize()
    torch.backends.cuda.matmul.allow_tf32 = False
    for shape in shapes:
        M, K, N = (int(v) for v in shape.split("x"))
        flop = roofline.gemm_flops(M, N, K)
        reps = max(5, min(200, int(0.15 / max(flop / 120e12, 1e-6))))

        def timeit(call):
            for _ in range(3):
                call()
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(reps)]
            for e0, e1 in ev:
                e0.record(stream)
                call()
                e1.record(stream)
            torch.cuda.synchronize()
            return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3

        C = torch.rand((M, N), device="cuda", generator=gen)
        for ta, tb in ((0, 0), (1, 0), (0, 1), (1, 1)):
            A = torch.rand((K, M) if ta else (M, K), device="cuda", generator=gen)
            B = torch.rand((N, K) if tb else (K, N), device="cuda", generator=gen)
            lda, ldb = A.shape[1], B.shape[1]
            need = binding.gemm_f32_general_workspace_bytes(ta, tb, M, N, K, lda, ldb)
            ws = torch.empty(max(need // 4, 1), device="cuda")
            res = []
            for alpha, beta in ((1.0, 0.0), (2.0, 0.5)):
                us = timeit(lambda: binding.gemm_f32_general(ta, tb, M, N, K, alpha, A, lda, B, ldb,
                                                             beta, C, N, ws, need,
                                                             stream.cuda_stream))
                res.append(us)
            opA = A.t() if ta else A
            opB = B.t() if tb else B
            t_v = timeit(lambda: torch.matmul(opA, opB, out=C))
            case = "NT"[ta] + "NT"[tb]
            print(f"{shape} {case}: alpha=1,beta=0 {res[0]:.1f} us ({flop / res[0] / 1e6:.1f} TF) | "
                  f"alpha=2,beta=0.5 {res[1]:.1f} us ({flop / res[1] / 1e6:.1f} TF) | "
                  f"vendor {t_v:.1f} us ({flop / t_v / 1e6:.1f} TF)", flush=True)
    return 0


def main(argv=None) -> int:
    import numpy as np
    import torch
    if argv and argv[0] == "--ladder":
        return ladder(np, torch)
    if argv and argv[0] == "--orders":
        return orders(np, torch, argv[1:] or ORDER_SHAPES)
    shapes = [tuple(int(x) for x in s.split("x")) for s in (argv or DEFAULT_SHAPES)]
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device="cuda").manual_seed(0)
    for (M, K, N) in shapes:
        dA = torch.rand((M, K), device="cuda", generator=gen) * 2 - 1
        dB = torch.rand((K, N), device="cuda", generator=gen) * 2 - 1
        dC = torch.empty((M, N), device="cuda")
        flop = roofline.gemm_flops(M, N, K)
        reps = max(5, min(200, int(0.15 / max(flop / 120e12, 1e-6))))

        def timeit(call):
            for _ in range(3):
                call()
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(reps)]
            for e0, e1 in ev:
                e0.record(stream)
                call()
                e1.record(stream)
            torch.cuda.synchronize()
            return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3

        def plan_call(plan):
            need = binding.gemm_f32_plan_workspace_bytes(M, N, K, plan)
            ws = torch.empty(max(need // 4, 1), device="cuda")
            return lambda: binding.gemm_f32_with_plan(dA, dB, dC, M, N, K, plan, ws, need,
                                                      stream.cuda_stream)

        res = []
        for kn in KERNELS:
            for sp in SPLITS:
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
                    if binding.gemm_f32_plan_workspace_bytes(M, N, K, plan) > MAX_WORKSPACE:
                        continue
                    res.append((timeit(plan_call(plan)), f"{kn}/{plan_label(plan)}"))
        auto = binding.gemm_f32_plan(M, N, K)
        t_auto = timeit(plan_call(auto))
        torch.backends.cuda.matmul.allow_tf32 = False
        t_vendor = timeit(lambda: torch.matmul(dA, dB, out=dC))
        res.sort()
        top = "  ".join(f"{name} {us:.1f}" for us, name in res[:4])
        print(f"{M}x{K}x{N}: auto {binding.gemm_kernel_name(auto.kernel)}/{plan_label(auto)} "
              f"{t_auto:.1f} us ({flop / t_auto / 1e6:.1f} TF) | vendor {t_vendor:.1f} us "
              f"({flop / t_vendor / 1e6:.1f} TF) | best {top}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))

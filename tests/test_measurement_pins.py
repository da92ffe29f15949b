"""The bench's work and traffic accounting against the pages' own figures (CPU only)."""
import os

import pytest

from fp32_gemm_07_amd import roofline

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _timing_rows():
    rows = []
    with open(os.path.join(GOLDEN, "page_measurements.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            shape, ver, ms, gflops = [x.strip() for x in line.split("|")]
            M, K, N = (int(x) for x in shape.split())
            rows.append((M, K, N, ver, float(ms), float(gflops)))
    return rows


def _worked_example():
    vals = {}
    with open(os.path.join(GOLDEN, "lesson10_worked_example.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                key, val, *_ = [x.strip() for x in line.split("|")]
                vals[key] = float(val)
    return vals


@pytest.mark.parametrize("row", _timing_rows(), ids=lambda r: f"{r[0]}x{r[1]}x{r[2]}-{r[3]}")
def test_flop_convention_reproduces_page_tables(row):
    M, K, N, _, ms, gflops = row
    implied = gflops * 1e9 * ms * 1e-3
    # the printed ms carries 3 decimals: half a unit of it bounds the error
    slack = gflops * 1e9 * 0.0005e-3 + 0.005e9 * ms * 1e-3
    assert abs(roofline.gemm_flops(M, N, K) - implied) <= slack


def test_lesson10_worked_example():
    w = _worked_example()
    n = 1024
    assert roofline.gemm_flops(n, n, n) == pytest.approx(w["flops"], rel=5e-4)
    naive = roofline.tiled_read_floats(n, n, n, 1, 1, 1)
    assert naive == w["naive_reads"]
    assert 4 * naive == pytest.approx(w["naive_bytes"], rel=5e-4)
    t16 = roofline.tiled_read_floats(n, n, n, 16, 16, 16)
    assert (n // 16) ** 2 == w["tiled16_tiles"] and n // 16 == w["tiled16_phases"]
    assert 16 * 16 * 2 == w["tiled16_floats_per_phase"]
    assert t16 == pytest.approx(w["tiled16_reads"], rel=5e-3)
    assert 4 * t16 == pytest.approx(w["tiled16_bytes"], rel=1e-5)
    assert naive / t16 == 16
    assert roofline.gemm_flops(n, n, n) / (4 * naive) == pytest.approx(w["naive_ai"])
    assert roofline.gemm_flops(n, n, n) / (4 * t16) == pytest.approx(w["tiled16_ai"])


def test_mi355x_peaks():
    derived = roofline.MI355X_CUS * roofline.MI355X_CLOCK_GHZ * roofline.FP32_MFMA_FLOP_PER_CLK_PER_CU / 1e3
    assert derived == pytest.approx(roofline.PEAK_FP32_MFMA_TFLOPS, rel=1e-3)
    assert roofline.ridge_flop_per_byte() == pytest.approx(19.66, rel=1e-3)


def test_compulsory_bytes_of_standing_workloads():
    assert roofline.compulsory_bytes(4096, 4096, 4096) == 201_326_592
    assert roofline.compulsory_bytes(512, 512, 131072) == 537_919_488
    assert roofline.compulsory_bytes(1001, 777, 513) == 6_759_564

"""bench.py's host-side logic (CPU only): the one-GPU guard, the HBM traffic
table keyed by kernel source, and the shader-clock table parser."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_traffic_is_tied_to_the_kernel_source(tmp_path, monkeypatch):
    w, k = "square_4096", "dma_mfma32_f32_256x256x16_w8_s3"
    m = bench.MEASURED_TRAFFIC[(w, k)]
    want = round(bench.FETCH_FACTOR * m["fetch_kib"] * 1024 + bench.WRITE_FACTOR * m["write_kib"] * 1024)
    # The committed table matches the committed source.
    assert bench.measured_traffic(w, k) == want
    # A changed source (any byte) voids it; so does an unmeasured pair.
    other = tmp_path / "gemm_kernels.hpp"
    other.write_bytes(open(bench.KERNEL_SOURCE, "rb").read() + b"\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(other))
    assert bench.measured_traffic(w, k) is None
    monkeypatch.undo()
    assert bench.measured_traffic(w, "valu_f32_64x64x16") is None


@pytest.mark.parametrize("text,want", [
    ("S: 113Mhz *\n0: 500Mhz\n1: 2400Mhz\n", (113.0, 2400.0)),   # idle, between levels
    ("0: 500Mhz\n1: 2400Mhz *\n", (2400.0, 2400.0)),             # at the top level
    ("S: 2312Mhz *\n0: 500Mhz\n1: 2400Mhz\n", (2312.0, 2400.0)),
    ("", (None, None)),
])
def test_shader_clock_table(tmp_path, text, want):
    p = tmp_path / "pp_dpm_sclk"
    p.write_text(text)
    assert bench.read_sclk(str(p)) == want
    assert bench.read_sclk(str(tmp_path / "absent")) == (None, None)


def test_cpu_sample_covers_every_row_when_time_allows():
    """The CPU baseline's slab is all of C when the oracle's calibrated rate
    finishes it within the bound (the five standing workloads on the box), so
    the ragged last tile row of 1001 x 513 x 777 is compared too; otherwise a
    bounded number of rows, at least one."""
    assert bench.cpu_sample_rows(1001, 1e4, 12.0) == 1001
    assert bench.cpu_sample_rows(4096, 4096 / 2.0, 12.0) == 4096
    assert bench.cpu_sample_rows(4096, 100.0, 12.0) == 1200
    assert bench.cpu_sample_rows(4096, 1e-3, 12.0) == 1


def test_settle_runs_steps_until_the_wall_time_has_passed():
    calls = []
    syncs = []
    el, n = bench.settle(lambda: calls.append(1), lambda: syncs.append(1), 5.0)
    assert el >= 5.0 and n == len(calls) >= 1
    # doubling batches, each ended by a synchronisation
    assert len(syncs) >= 1 and n == 2 ** len(syncs) - 1 or n >= 4096


def test_shapes_parse_as_m_k_n():
    assert bench.parse_shape("1001x513x777") == (1001, 513, 777)
    assert all(len(bench.parse_shape(s)) == 3 for s in bench.SWEEP_SHAPES + bench.ORDER_SHAPES)
    assert bench.LADDER_SHAPES == ["1024x512x1024", "1001x513x777"]

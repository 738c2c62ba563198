"""bench.py's host logic without a GPU: the multi-GPU refusal, the algorithmic
figures, the traffic lookup keyed by the source hash and the CPU baseline leg."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from dense_fp16_gemm_03_amd import inputs  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_shape_parsing():
    assert bench.parse_shape("4096x4096x1001") == (4096, 4096, 1001)
    for bad in ("8192^3", "4096x4096", "0x5x5", "axbxc", "1x2x-3"):
        assert bench.parse_shape(bad) is None


def test_shard_shapes_are_one_gpus_share():
    """The shard shapes are 1/8 of a workload: M/8 of 8192^3 (same N and K),
    K/8 of each long-K workload (same M and N); every timed shape has a call
    count."""
    W = inputs.WORKLOADS
    for name, (m, n, k) in inputs.SHARD_SHAPES.items():
        base, split = name.split(" ")
        M, N, K = W[base]
        assert (split, (m, n, k)) in (("M/8", (M // 8, N, K)), ("K/8", (M, N, K // 8)))
        assert 2 * m * n * k * 8 == 2 * M * N * K
    for table in (W, inputs.PAGE_SHAPES, inputs.SHARD_SHAPES):
        assert all(name in bench.CALLS for name in table)


def test_algorithmic_figures():
    flops, nbytes = bench.algorithmic(8192, 8192, 8192)
    assert flops == 2.0 * 8192**3
    assert nbytes == 2.0 * (2 * 8192 * 8192) + 4.0 * 8192 * 8192  # A, B read once, C written once
    assert bench.algorithmic(1024, 1024, 65536) == (2.0 * 1024 * 1024 * 65536,
                                                    2.0 * 2 * 1024 * 65536 + 4.0 * 1024 * 1024)


def test_traffic_needs_the_current_source(tmp_path, monkeypatch):
    good = tmp_path / "traffic.json"
    good.write_text(json.dumps({"8192^3": {"source_hash": bench.source_hash(),
                                           "bytes_per_launch": 123}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(good))
    assert bench.traffic_for("8192^3") == 123
    assert bench.traffic_for("1024^3") is None
    stale = tmp_path / "stale.json"
    stale.write_text(json.dumps({"8192^3": {"source_hash": "0" * 16, "bytes_per_launch": 123}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(stale))
    assert bench.traffic_for("8192^3") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_for("8192^3") is None


def test_cpu_baseline_record():
    M, N, K = 64, 48, 32
    A, B = inputs.uniform(M, K, 1), inputs.uniform(N, K, 2)
    r = bench.cpu_baseline(A, B, M, N, K, budget_s=0.05)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["cores"] >= 1
    assert r["value"] > 0 and "rows 0.." in r["sample"]
    Ab = inputs.uniform_bf16(M, K, 1)
    Bb = inputs.uniform_bf16(N, K, 2)
    assert np.isfinite(bench.cpu_baseline(Ab, Bb, M, N, K, budget_s=0.05)["value"])


def test_roofline_bound_per_config():
    """256^3 and 1024^3 sit below the ridge (HBM-bound); the other three
    workloads are MFMA-bound."""
    bounds = {n: bench.roofline_time(*inputs.WORKLOADS[n])[1] for n in inputs.WORKLOADS}
    assert bounds == {"256^3": "hbm", "1024^3": "hbm", "2048x2048x16384": "mfma",
                      "1024x1024x65536": "mfma", "8192^3": "mfma"}
    t, _ = bench.roofline_time(8192, 8192, 8192)
    assert abs(t - 2.0 * 8192**3 / 2.5e15) < 1e-12
    t, _ = bench.roofline_time(1024, 1024, 1024)
    assert abs(t - (2.0 * 2 * 1024 * 1024 + 4.0 * 1024 * 1024) / 8e12) < 1e-15


def test_clock_window_summary():
    """The telemetry summary keeps only the samples inside the timed window
    and reads the power-limit residency as the ratio of counter deltas."""
    s = bench.ClockSampler.__new__(bench.ClockSampler)
    s.samples = [(0.5, [2400] * 8, 900, 0, 0, 0),
                 (1.0, [1600] * 8, 1400, 100, 1000, 5),
                 (1.5, [1700, 1500] * 4, 1380, 500, 2000, 9),
                 (3.0, [2400] * 8, 800, 600, 3000, 12)]
    w = s.window(0.9, 2.0)
    assert w["samples"] == 2
    assert w["gfx_clk_mhz_mean"] == 1600.0
    assert w["gfx_clk_mhz_per_xcd"] == [1650.0, 1550.0] * 4
    assert w["ppt_limited_frac"] == 0.4  # (500 - 100) / (2000 - 1000)
    assert s.window(5.0, 6.0) is None


def test_fraction_at_a_clock():
    """The peak scales with the shader clock: 2.5 PF at 2400 MHz, half of it
    at 1200 MHz."""
    flops = 2.0 * 8192 ** 3
    us = flops / (bench.PEAK_TFLOPS * 1e12) * 1e6
    assert bench.frac_at_clock(flops, us, bench.PEAK_SCLK_MHZ) == 1.0
    assert bench.frac_at_clock(flops, 2 * us, bench.PEAK_SCLK_MHZ / 2) == 1.0
    assert bench.frac_at_clock(flops, 2 * us, bench.PEAK_SCLK_MHZ) == 0.5

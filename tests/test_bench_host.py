"""Host logic of bench.py that the line's measured fields rest on (CPU only): the clock/power summary of the
amdsmi samples, and the reading of the harness's machine-readable summary lines, which are taken only for the
kernel build and workload they name."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_clock_power_summary_drops_the_lagging_start_and_scales_the_peak():
    s = bench.ClockPowerSampler()
    s.limit_w = 1400.0
    # (time, mean clock over the XCDs, lowest XCD, highest XCD, socket power): the first second still shows idle
    s.samples = [(0.0, 150.0, 140, 160, 260.0), (0.5, 150.0, 140, 160, 260.0)]
    s.samples += [(1.0 + 0.1 * i, 1700.0 + (i % 2) * 20.0, 1650, 1790, 1340.0 + i) for i in range(10)]
    out = s.summary("a test run", achieved_tflops=1200.0, skip_s=0.8)
    assert out["samples"] == 10
    assert out["gfxclk_mhz_mean"] == pytest.approx(1710.0)
    assert (out["gfxclk_mhz_xcd_min"], out["gfxclk_mhz_xcd_max"]) == (1650, 1790)
    assert out["socket_power_w_mean"] == pytest.approx(1344.5)
    assert out["socket_power_w_max"] == 1349.0 and out["power_limit_w"] == 1400.0
    peak = bench.BF16_PEAK_TFLOPS * 1710.0 / bench.NOMINAL_SCLK_MHZ
    assert out["bf16_peak_at_sampled_clock_tflops"] == pytest.approx(peak, abs=0.05)
    assert out["frac_at_sampled_clock"] == pytest.approx(1200.0 / peak, abs=1e-4)


def test_clock_power_summary_without_samples_reports_the_error():
    s = bench.ClockPowerSampler()
    s.error = "AmdSmiLibraryException: driver not loaded"
    out = s.summary("a test run", achieved_tflops=1200.0, skip_s=0.8)
    assert out["samples"] == 0 and "driver not loaded" in out["error"]
    assert "gfxclk_mhz_mean" not in out


def _summary(path, sha, workload):
    with open(path, "w") as f:
        f.write("# a summary\n\n| launch | x |\n|---|---|\n| 0 | 1 |\n\n    a command: with a colon\n\n")
        f.write(f"kernel_build_sha256: {sha}\nworkload: {workload}\nhbm_bytes_per_launch: 1.25e+09\n")


def test_summary_fields_are_taken_only_for_this_build_and_workload(tmp_path):
    from exact_blockwise_attention_fwd_amd.build import fingerprint

    w = W.WORKLOADS["ring_share_128k"]
    sha = fingerprint(os.path.basename(bench.FWD_SOURCE))
    good = tmp_path / "good.txt"
    _summary(good, sha, w.name)
    f = bench.recorded_fields(str(good), w)
    assert f is not None and float(f["hbm_bytes_per_launch"]) == 1.25e9
    other_build = tmp_path / "other_build.txt"
    _summary(other_build, "0" * 64, w.name)
    assert bench.recorded_fields(str(other_build), w) is None
    other_workload = tmp_path / "other_workload.txt"
    _summary(other_workload, sha, "causal_prefill_4k")
    assert bench.recorded_fields(str(other_workload), w) is None
    assert bench.recorded_fields(str(tmp_path / "missing.txt"), w) is None

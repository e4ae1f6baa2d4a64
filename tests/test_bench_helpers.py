"""bench.py's host-side helpers on the CPU: the roofline object, the oracle baselines of
the bench lines (on tiny samples), and the lookup of recorded counter traffic."""
import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from combine_dispatch_layout_amd import workloads  # noqa: E402


def test_hbm_roofline_fields():
    r = bench.hbm_roofline("combine", 8e9, 1000.0, traffic=8.1e9, M=4)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["kernel"] == "combine"
    assert r["achieved"] == pytest.approx(8000.0) and r["peak"] == bench.HBM_PEAK_GBPS
    assert r["frac"] == pytest.approx(1.0)
    assert r["traffic"] == 8.1e9 and r["alg_bytes_per_launch"] == 8_000_000_000
    assert r["launch_us"] == 1000.0 and r["M"] == 4


def _check_baseline(c, unit):
    assert c["kind"] == "oracle" and c["cores"] == 1 and c["unit"] == unit
    assert c["value"] > 0 and c["seconds"] >= 0 and c["sample"]


def test_cpu_small_baseline():
    c = bench.cpu_small_baseline(workloads.make_workload(1, M=8), seconds=0.0)
    _check_baseline(c, "us")
    assert "M=8" in c["sample"]


def test_cpu_bucket_baseline():
    w = workloads.make_workload(3, M=32)
    c = bench.cpu_bucket_baseline(w, 16)
    _check_baseline(c, "GB/s")
    assert "first 16 tokens" in c["sample"]
    assert set(c["phase_seconds"]) == {"layout", "dispatch", "expand", "combine_partial",
                                       "combine_reduce"}


class _Weights:
    """Stands in for the device weight stack: builds only the experts asked for."""

    def __init__(self, nout, k):
        self.nout, self.k = nout, k

    def __getitem__(self, experts):
        g = torch.Generator().manual_seed(3)
        return (torch.randn((len(experts), self.nout, self.k), generator=g) * 0.02).to(
            torch.bfloat16).view(torch.int16)


def test_cpu_gemm_baseline():
    w = workloads.make_workload(3, M=16)
    c = bench.cpu_gemm_baseline(w, _Weights(128, w.N), 128, 40)
    _check_baseline(c, "TFLOP/s")
    assert c["sample"].startswith(f"first 40 of {w.M * w.k} rows")


def test_recorded_traffic(tmp_path):
    good = tmp_path / "good.txt"
    sha = bench.source_hash(bench.KERNEL_SOURCES["expand"])
    good.write_text("# comment: ignored\nworkload: wl\n"
                    f"expand.source_sha256: {sha}\nexpand.hbm_bytes_per_launch: 123\n")
    assert bench.recorded_traffic("expand", "wl", str(good)) == 123.0
    assert bench.recorded_traffic("expand", "other", str(good)) is None      # workload
    stale = tmp_path / "stale.txt"
    stale.write_text("workload: wl\nexpand.source_sha256: 0000\n"
                     "expand.hbm_bytes_per_launch: 123\n")
    assert bench.recorded_traffic("expand", "wl", str(stale)) is None        # source changed
    assert bench.recorded_traffic("expand", "wl", str(tmp_path / "missing.txt")) is None


def test_committed_profiles_parse():
    """Every committed counter summary names its workload and, per kernel, a source hash
    and a byte count; those taken on the current sources give a positive traffic figure
    (a summary left behind by a kernel change gives none, which is allowed)."""
    for name in sorted(os.listdir(bench.PROFILES)):
        if not name.startswith("hbm_traffic_"):
            continue
        wl = name[len("hbm_traffic_"):-len(".txt")]
        text = open(os.path.join(bench.PROFILES, name)).read()
        assert f"workload: {wl}" in text
        for kernel in bench.KERNEL_SOURCES:
            if f"{kernel}.hbm_bytes_per_launch:" in text:
                assert f"{kernel}.source_sha256:" in text
                t = bench.recorded_traffic(kernel, wl, os.path.join(bench.PROFILES, name))
                assert t is None or t > 0


def test_event_steps():
    """The timed loop records per-kernel events on a few evenly spaced steps: every step
    when there are few of them, never one outside [0, K), and not the first step once
    there are ten or more."""
    assert bench.event_steps(3) == [0, 1, 2]
    assert bench.event_steps(5) == [0, 1, 2, 3, 4]
    assert bench.event_steps(20) == [2, 6, 10, 14, 18]
    assert bench.event_steps(100) == [10, 30, 50, 70, 90]
    for K in range(1, 300):
        s = bench.event_steps(K)
        assert all(0 <= i < K for i in s) and len(s) == min(K, 5)
        assert s == sorted(set(s))
        if K >= 10:
            assert s[0] > 0

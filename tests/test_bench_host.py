"""Host-side logic of bench.py (no GPU): the rule that ties a committed
traffic summary to the kernel sources it was measured with, the least-squares
line of the linearity check, and the --gpus contract."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench


def _summary(path, workload, entry, digest, traffic):
    path.write_text(f"# HBM traffic\n\nworkload: {workload}\nentry point: {entry}\n"
                    f"kernel sources sha256: {digest}\ntraffic bytes per launch: {traffic}\n")


def test_traffic_counts_only_for_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_GLOB", str(tmp_path / "vmm_traffic_*.md"))
    wl, entry = "llama3-8b-gate-4096x14336-avg3", bench.ENTRY["accumulate"]
    _summary(tmp_path / "vmm_traffic_a.md", wl, entry, "0" * 64, 123.0)
    assert bench.measured_traffic(wl, "accumulate") is None          # older sources: ignored
    _summary(tmp_path / "vmm_traffic_b.md", wl, entry, bench.kernel_source_hash(), 456.0)
    assert bench.measured_traffic(wl, "accumulate") == 456.0
    assert bench.measured_traffic(wl, "decode") is None               # other entry point
    assert bench.measured_traffic("attn-proj-4096x4096-avg3", "accumulate") is None


def test_source_hash_covers_the_vmm_sources():
    assert len(bench.kernel_source_hash()) == 64
    for rel in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(bench.ROOT, rel)), rel


def test_linear_fit_recovers_a_line():
    bw = 7.5e3                                       # GB/s
    pts = [(b, 16.0 + b / (bw * 1e3)) for b in (2e7, 5e7, 1e8, 2.4e8)]
    fit = bench.linear_fit(pts)
    assert fit["intercept_us"] == pytest.approx(16.0, rel=1e-9)
    assert fit["bw_eff_GB_s"] == pytest.approx(bw, rel=1e-9)
    assert fit["r2"] == pytest.approx(1.0)
    noisy = [(b, t + (0.5 if i % 2 else -0.5)) for i, (b, t) in enumerate(pts)]
    assert bench.linear_fit(noisy)["r2"] < 1.0


def test_workloads_are_consistent():
    for name, (K, N, cfg, mat, key, lv) in bench.WORKLOADS.items():
        P, levels = bench._P(key, lv)
        assert abs(sum(P) - 1.0) < 1e-9 and len(P) == len(levels), name
        assert max(levels) <= bench.bmax_of(lv), name
    assert bench.DEFAULT in bench.WORKLOADS


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_rotation_is_sized_by_bytes_read():
    """One cycle through the copies reads at least 512 MiB (twice the 256 MB
    Infinity Cache), counting the bytes a step reads, not the store's size."""
    for step_bytes in (4.72e6, 16.4e6, 23.76e6, 22.5e6, 242e6, 6e8):
        R = bench.rotation_copies(step_bytes)
        assert R * step_bytes >= bench.ROT_BYTES
        assert (R - 1) * step_bytes < bench.ROT_BYTES or R == 2
        assert R <= bench.MAX_COPIES
    assert bench.rotation_copies(23.76e6) == 23

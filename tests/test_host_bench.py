"""Host logic of bench.py: the lm head's roofline from launch rows and
times, the counter summaries keyed to the kernel sources, and the refusal of
more than one GPU.  No GPU."""
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

import bench

H, V = 3840, 262144


def test_head_roofline_mfma_launches():
    M, ms = [2210] * 5, [3.5, 3.4, 3.6, 3.5, 3.5]
    r = bench.head_roofline(M, ms, H, V)
    flops = 2.0 * H * V * 2210 * 5
    ach = flops / (sum(ms) * 1e-3) / 1e12
    assert r["bound"] == "mfma" and r["roof"]["unit"] == "TFLOP/s"
    assert r["roof"]["achieved"] == pytest.approx(ach, abs=0.01)
    assert r["roof"]["frac"] == pytest.approx(ach / 2500.0, abs=1e-4)
    assert list(r["bounds"]) == ["mfma"] * 5
    # every launch on one bound: the time-weighted figure is the aggregate
    assert r["time_weighted_frac"] == pytest.approx(r["roof"]["frac"], abs=1e-4)


def test_head_roofline_never_mixes_bounds():
    # one MFMA-bound launch (560 rows) and two HBM-bound ones (280 rows) that
    # hold most of the time: the figure is HBM, over those two launches only
    M, ms = [560, 280, 280], [1.0, 0.7, 0.7]
    r = bench.head_roofline(M, ms, H, V)
    assert list(r["bounds"]) == ["mfma", "hbm", "hbm"]
    assert r["bound"] == "hbm" and r["roof"]["unit"] == "GB/s"
    nbytes = 2.0 * H * V + 280 * H * 2.0
    gbs = 2 * nbytes / (1.4e-3) / 1e9
    assert r["roof"]["achieved"] == pytest.approx(gbs, abs=0.1)
    assert r["roof"]["frac"] == pytest.approx(gbs / 8000.0, abs=1e-4)
    # per-launch fractions, each against its own bound
    f0 = 2.0 * H * V * 560 / 1e-3 / 1e12 / 2500.0
    assert r["fracs"][0] == pytest.approx(f0, rel=1e-9)
    tw = (f0 * 1.0 + 2 * (nbytes / 0.7e-3 / 1e9 / 8000.0) * 0.7) / 2.4
    assert r["time_weighted_frac"] == pytest.approx(tw, abs=1e-4)


def test_head_roofline_ridge():
    # 2.5 PFLOP/s over 8 TB/s: 312.5 flop per W byte, i.e. scored rows per W stream
    assert bench.HEAD_RIDGE_ROWS == pytest.approx(312.5)
    r = bench.head_roofline([312, 313], [1.0, 1.0], H, V)
    assert list(r["bounds"]) == ["hbm", "mfma"]


def _tree(tmp_path):
    for kernel, files in bench.KERNEL_SOURCES.items():
        for f in files:
            dst = tmp_path / f
            dst.parent.mkdir(parents=True, exist_ok=True)
            shutil.copy(os.path.join(bench.HERE, f), dst)
    (tmp_path / "profiles").mkdir()


def test_traffic_summary_keyed_to_sources(tmp_path, monkeypatch):
    _tree(tmp_path)
    monkeypatch.setattr(bench, "HERE", str(tmp_path))
    assert bench.measured_traffic("head_lse_kernel", "moderation") == (None, "no counter summary for moderation")
    h = bench.source_hash("head_lse_kernel")
    p = tmp_path / "profiles" / "head_lse_kernel_moderation_traffic.md"
    p.write_text(f"# t\n\nsource_sha256: {h}\nhbm_bytes_per_launch[per_launch]: 123456789\n")
    assert bench.measured_traffic("head_lse_kernel", "moderation") == (123456789.0,
                                                                      "profiles/head_lse_kernel_moderation_traffic.md")
    p.write_text("# t\n\nno figures\n")
    assert bench.measured_traffic("head_lse_kernel", "moderation")[0] is None
    # an edit of any file that defines the kernel voids the summary
    p.write_text(f"# t\n\nsource_sha256: {h}\nhbm_bytes_per_launch[per_launch]: 123456789\n")
    with open(tmp_path / bench.KERNEL_SOURCES["head_lse_kernel"][1], "a") as fh:
        fh.write("\n")
    assert bench.measured_traffic("head_lse_kernel", "moderation") == (
        None, "kernel changed since the counters were taken")


def test_shared_header_keys_both_kernels(tmp_path, monkeypatch):
    _tree(tmp_path)
    monkeypatch.setattr(bench, "HERE", str(tmp_path))
    shared = set(bench.KERNEL_SOURCES["head_lse_kernel"]) & set(bench.KERNEL_SOURCES["branch_attention"])
    assert shared
    before = {k: bench.source_hash(k) for k in bench.KERNEL_SOURCES}
    with open(tmp_path / sorted(shared)[0], "a") as fh:
        fh.write("\n")
    assert all(bench.source_hash(k) != before[k] for k in bench.KERNEL_SOURCES)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.HERE, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr

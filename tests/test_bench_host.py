"""Host-side parts of bench.py: the one-GPU guard and the readers of the
committed rocprofv3 summaries (no GPU is touched)."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def _write(root, name, lines):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    with open(os.path.join(root, "profiles", name), "w") as f:
        f.write("\n".join(lines) + "\n")


COUNTER_LINES = ["# header", "kernel_source_sha256_16: abc", "algorithmic_flops_per_launch: 100",
                 "auto.mfma_busy_pct: 30.5", "auto.valu_busy_pct: 57.0",
                 "auto.mfma_valu_coexec_pct: 34.0", "auto.mfma_f16_flops_per_launch: 105",
                 "auto.mfma_f16_flops_over_algorithmic: 1.05"]


def test_counter_summary_is_read_for_its_precision(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc")
    _write(str(tmp_path), "attention_fwd_wl_mfma.txt", COUNTER_LINES)
    got = bench.read_counters("wl", "auto")
    assert got["mfma_busy_pct"] == 30.5 and got["mfma_f16_flops_over_algorithmic"] == 1.05
    assert got["source"] == os.path.join("profiles", "attention_fwd_wl_mfma.txt")
    assert bench.read_counters("wl", "fast") is None      # no block for that precision
    assert bench.read_counters("other", "auto") is None   # no file


def test_summaries_of_another_kernel_source_are_ignored(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "def")
    _write(str(tmp_path), "attention_fwd_wl_mfma.txt", COUNTER_LINES)
    _write(str(tmp_path), "attention_fwd_wl_traffic.txt",
           ["kernel_source_sha256_16: abc", "hbm_bytes_per_launch: 1234"])
    assert bench.read_counters("wl", "auto") is None
    assert bench.read_traffic("wl") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc")
    assert bench.read_traffic("wl") == 1234


@pytest.mark.parametrize("name", sorted(os.listdir(os.path.join(ROOT, "profiles"))))
def test_committed_summaries_carry_their_kernel_hash_and_command(name):
    text = open(os.path.join(ROOT, "profiles", name)).read()
    assert "kernel_source_sha256_16:" in text
    assert "rocprofv3 " in text and "python bench.py" in text


def test_replay_plan_times_exactly_the_requested_steps():
    for steps in (1, 5, 7, 20, 30, 50, 97, 100, 1000):
        r, g = bench.replay_plan(steps)
        assert r * g == steps and 1 <= r <= 10
        assert g >= min(10, steps)          # no graph of a couple of launches
    assert bench.replay_plan(50) == (5, 10)
    assert bench.replay_plan(20) == (2, 10)
    assert bench.replay_plan(100) == (10, 10)
    assert bench.replay_plan(1000) == (10, 100)
    assert bench.replay_plan(7) == (1, 7)
    assert bench.replay_plan(97) == (1, 97)


def test_roofline_bound_follows_the_ridge():
    import workloads
    kinds = {w.wid: bench.roofline_bound(w.flops, w.algorithmic_bytes)
             for w in workloads.WORKLOADS.values()}
    # 4*H*N^2*d flop over 16*H*N*d bytes = N/4 flop per byte; ridge ~315
    assert kinds[1] == kinds[2] == kinds[3] == "hbm"
    assert kinds[4] == kinds[5] == "mfma"
    assert abs(bench.RIDGE_FLOP_PER_BYTE - 314.575) < 1e-3


def test_percentile():
    xs = [5.0, 1.0, 3.0, 2.0, 4.0]
    assert bench.percentile(xs, 50) == 3.0
    assert bench.percentile(xs, 0) == 1.0 and bench.percentile(xs, 100) == 5.0
    assert abs(bench.percentile(xs, 10) - 1.4) < 1e-12
    assert bench.percentile([7.0], 90) == 7.0

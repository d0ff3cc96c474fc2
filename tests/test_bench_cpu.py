"""Host-side logic of bench.py, no GPU: the one-GPU guard, the hash gate on
the committed PMC traffic figure and the clock report's plausibility flag."""
import json
import os
import subprocess
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def _write_traffic(path, khash, hbm):
    with open(path, "w") as f:
        f.write("# traffic summary\n")
        f.write(f"kernel_source_sha256_16 = {khash}\n")
        f.write(f"hbm_bytes_per_launch = {hbm}\n")


def test_traffic_is_reported_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    path = str(tmp_path / "traffic.txt")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", path)
    assert bench._traffic() is None                       # no file
    _write_traffic(path, bench._kernel_hash(), 7046733636)
    assert bench._traffic() == 7046733636.0
    _write_traffic(path, "0" * 16, 7046733636)             # counters of another source
    assert bench._traffic() is None
    with open(path, "w") as f:
        f.write(f"kernel_source_sha256_16 = {bench._kernel_hash()}\n")
    assert bench._traffic() is None                       # no figure in the file


def test_kernel_hash_follows_the_attention_sources(tmp_path, monkeypatch):
    a, b = tmp_path / "a.hip", tmp_path / "b.h"
    a.write_text("kernel one\n")
    b.write_text("helpers\n")
    monkeypatch.setattr(bench, "ATTN_KERNEL_SRCS", [str(a), str(b)])
    h1 = bench._kernel_hash()
    a.write_text("kernel two\n")
    assert bench._kernel_hash() != h1 and len(h1) == 16


def test_clock_report_flags_readings_below_the_rate(monkeypatch):
    monkeypatch.setattr(bench, "torch", torch, raising=False)
    c = bench.ClockSampler()                    # no GPU here: amdsmi is not used
    # the first (pre-load) reading is dropped; 1300 TFLOP/s needs >= 1248 MHz
    c.metrics = [100.0] + [1650.0] * 20
    c.clk = [100.0] + [150.0] * 20
    rep = c.report(1300.0)
    assert rep["min_clock_mhz_for_rate"] == 1248.0
    m, k = rep["gpu_metrics_current_gfxclk"], rep["clock_info_gfx"]
    assert m["median_mhz"] == 1650.0 and m["plausible"] and m["representative"]
    assert k["median_mhz"] == 150.0 and not k["plausible"]
    c.metrics = [100.0, 1650.0, 1650.0]         # a short window: not representative
    assert not c.report(1300.0)["gpu_metrics_current_gfxclk"]["representative"]
    c.metrics = []
    assert c.report()["gpu_metrics_current_gfxclk"]["samples"] == 0

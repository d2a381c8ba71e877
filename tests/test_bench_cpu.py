"""bench.py's host logic on the CPU: the one-GPU rule, and the roofline entry
with its counter traffic, which counts only when the counters were taken on
the sources as they are now."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _counters(tmp_path, monkeypatch, src_bytes, recorded_sha):
    src = tmp_path / "kernel.hip"
    src.write_bytes(src_bytes)
    js = {"stage_c2": {"hbm_bytes_per_call": 32.5e6,
                       "sources": {os.path.relpath(src, bench.ROOT): recorded_sha}}}
    path = tmp_path / "hbm_counters.json"
    path.write_text(json.dumps(js))
    monkeypatch.setattr(bench, "COUNTERS", str(path))


def test_traffic_counts_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    body = b"__global__ void k() {}\n"
    _counters(tmp_path, monkeypatch, body, hashlib.sha256(body).hexdigest())
    assert bench.counters_traffic("stage_c2") == pytest.approx(32.5e6)
    assert bench.counters_traffic("no_such_entry") is None


def test_traffic_is_null_once_a_source_changed(tmp_path, monkeypatch):
    _counters(tmp_path, monkeypatch, b"changed\n", hashlib.sha256(b"original\n").hexdigest())
    assert bench.counters_traffic("stage_c2") is None


def test_roofline_entry_fields(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "COUNTERS", str(tmp_path / "missing.json"))
    r = bench.roofline_entry("stage_c2", 26215200, 31.4, "selection stage", {"extra": 1})
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.HBM_PEAK_GBS
    assert r["achieved"] == pytest.approx(26215200 / 31.4e-6 / 1e9)
    assert r["frac"] == pytest.approx(r["achieved"] / bench.HBM_PEAK_GBS)
    assert r["traffic"] is None  # no counter file
    assert r["bytes_per_call"] == 26215200 and r["us_per_call"] == 31.4 and r["extra"] == 1

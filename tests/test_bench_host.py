"""Host-side logic of bench.py (no GPU): the one-GPU guard, the HBM traffic
taken from the committed counter readings, and the oracle baseline's report."""

import json
import os
import subprocess
import sys

import bench
from workloads import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _counters(tmp_path, source_hash):
    c = {"kernel_source_sha256_16": source_hash,
         "workloads": {"qwen05": {"fwd": {"fetch_kib": 10.0, "write_kib": 20.0},
                                  "bwd": {"fetch_kib": 100.0, "write_kib": 50.0},
                                  "finalize": {"fetch_kib": 3.0, "write_kib": 1.0}}},
         "copy_calibration": {"fetch_scale": 2.0, "write_scale": 1.0}}
    p = tmp_path / "counters.json"
    p.write_text(json.dumps(c))
    return str(p)


def test_traffic_is_the_backward_calls_scaled_counter_bytes(tmp_path, monkeypatch):
    w = configs.get("qwen05")
    monkeypatch.setattr(bench, "COUNTERS", _counters(tmp_path, bench.kernel_hash()))
    # (100 * 2 + 50 * 1) + (3 * 2 + 1 * 1) KiB: main kernel plus the dw finalize
    assert bench.traffic_from_counters("qwen05", w) == (250 + 7) * 1024.0
    assert bench.traffic_from_counters("7b", configs.get("7b")) is None


def test_traffic_is_null_for_another_kernel_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "COUNTERS", _counters(tmp_path, "0" * 16))
    assert bench.traffic_from_counters("qwen05", configs.get("qwen05")) is None
    monkeypatch.setattr(bench, "COUNTERS", str(tmp_path / "missing.json"))
    assert bench.traffic_from_counters("qwen05", configs.get("qwen05")) is None


def test_cpu_baseline_report(oracle_mod):
    r = bench.cpu_baseline(configs.get("tiny"), 0.2)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s"
    assert r["value"] > 0 and r["cores"] >= 1
    assert r["single_thread"]["value"] > 0
    assert "tiny" in r["sample"] and "threads" in r["sample"]

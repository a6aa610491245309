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
    monkeypatch.setattr(bench, "COUNTERS", _counters(tmp_path, bench.kernel_hash()))
    # (100 * 2 + 50 * 1) + (3 * 2 + 1 * 1) KiB: main kernel plus the dw finalize
    assert bench.traffic_from_counters("qwen05") == (250 + 7) * 1024.0
    assert bench.traffic_from_counters("7b") is None


def test_traffic_is_null_for_another_kernel_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "COUNTERS", _counters(tmp_path, "0" * 16))
    assert bench.traffic_from_counters("qwen05") is None
    monkeypatch.setattr(bench, "COUNTERS", str(tmp_path / "missing.json"))
    assert bench.traffic_from_counters("qwen05") is None


def test_cpu_baseline_report(oracle_mod):
    """The oracle's report: forward and backward timed apart on every core the
    process may use, one-thread runs, the CPU model, and the host BFD packer on
    both document mixes with their bin counts."""
    w = configs.get("tiny")
    r = bench.cpu_baseline(w, 0.2)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s"
    assert r["value"] > 0 and r["cores"] == len(os.sched_getaffinity(0))
    assert r["cpu_model"]
    for part in ("fwd", "bwd"):
        assert r[part]["ms"] > 0 and r[part]["GBps_equiv"] > 0
    assert abs(r["value"] - w.tokens / ((r["fwd"]["ms"] + r["bwd"]["ms"]) * 1e-3)) < 1e-3 * r["value"]
    assert r["single_thread"]["tiny"]["fwd_bwd_tokens_per_s"] > 0
    assert "tiny" in r["sample"] and "threads" in r["sample"]
    for mix in r["bfd_pack"].values():
        assert mix["status"] == 0 and mix["bins"] >= 1 and mix["us"] > 0
    assert "parity" not in r


def test_cpu_baseline_parity_of_given_outputs(oracle_mod):
    """With host copies of outputs, the report carries their parity statistics
    against the oracle; the oracle's own (rounded) outputs pass with zero
    error, and a planted error is reported as a failure instead of raising."""
    import numpy as np

    import oracle
    from workloads import gen

    w = configs.get("tiny")
    inp = gen.make_inputs(w, backward=True)
    dec = lambda a: oracle.decode(a, w.dtype)  # noqa: E731
    a = (w.rotary_dim, w.eps, w.theta)
    yq, yk = oracle.fwd(dec(inp["q"]), dec(inp["k"]), dec(inp["wq"]), dec(inp["wk"]), inp["pos"], *a)
    g = oracle.bwd(dec(inp["q"]), dec(inp["k"]), dec(inp["wq"]), dec(inp["wk"]), inp["pos"],
                   dec(inp["dyq"]), dec(inp["dyk"]), *a)
    out = {key: v.astype(np.float32) for key, v in
           zip(("yq", "yk", "dq", "dk", "dwq", "dwk"), (yq, yk) + tuple(g))}
    r = bench.cpu_baseline(w, 0.2, out)
    assert set(r["parity"]) >= {"yq", "yk", "dq", "dk", "dwq", "dwk", "rule"}
    assert all(r["parity"][key]["max_abs"] < 1e-6 for key in ("yq", "yk", "dq", "dk"))
    out["dk"] = out["dk"].copy()
    out["dk"][0, 0, 0] += 1e-3
    r = bench.cpu_baseline(w, 0.2, out)
    assert "fail" in r["parity"]["dk"] and "fail" not in r["parity"]["dq"]

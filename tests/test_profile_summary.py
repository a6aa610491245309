"""Host logic of profile_summary.py (no GPU): kernel names, the phases of a
bench run told apart by dispatch order, and the counter file bench.py reads,
on small synthetic rocprofv3 CSVs."""

import csv
import json
import os

import profile_summary as ps

QK = "void (anonymous namespace)::qknr_kernel<(anonymous namespace)::Bf16, 64, 2, %s, false, false, false>((anonymous namespace)::Params)"
FIN = "void (anonymous namespace)::qknr_dw_finalize_kernel<(anonymous namespace)::Bf16>(float const*, int, int, (anonymous namespace)::GradCols)"
FLUSH = "(anonymous namespace)::bench_flush_kernel(unsigned int __vector(4)*, long, unsigned int)"
COPY = "(anonymous namespace)::bench_copy_kernel(unsigned int __vector(4) const*, unsigned int __vector(4)*, long)"
EMPTY = "(anonymous namespace)::bench_empty_kernel()"
GW = "void (anonymous namespace)::qknr_gwave_kernel<(anonymous namespace)::Bf16, 128, true, false, false>((anonymous namespace)::Params)"
OTHER = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<long>>()"


def test_friendly_names():
    assert ps.friendly(QK % "false") == "qknr_kernel<bf16, D=64, fwd>"
    assert ps.friendly(QK % "true") == "qknr_kernel<bf16, D=64, bwd>"
    assert ps.friendly(FIN) == "qknr_dw_finalize_kernel"
    assert ps.friendly(GW) == "qknr_gwave_kernel<bf16, D=128, bwd>"
    assert ps.friendly(FLUSH) == ps.FLUSH and ps.friendly(COPY) == ps.COPY
    assert ps.friendly(EMPTY) == ps.EMPTY
    assert ps.friendly(OTHER) is None


# a bench run in miniature: steady-state fwd/bwd(+finalize), then cold calls
# after flushes, then the copies, then graph-replayed variants with the decode
# floor probes (an empty kernel, a small copy) among them
SEQ = [OTHER, QK % "false", QK % "true", FIN, QK % "false", QK % "true", FIN,
       FLUSH, QK % "false", FLUSH, QK % "true", FIN,
       FLUSH, COPY, COPY, GW, FIN, EMPTY, COPY, GW]


def _write_trace(d, seq):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_kernel_trace.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp",
                    "LDS_Block_Size", "Workgroup_Size_X", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"])
        t = 1000
        for i, n in enumerate(seq, 1):
            w.writerow(["KERNEL_DISPATCH", i, n, t, t + 1000 * i, 0, 256, 1024, 1, 1])
            t += 100000


def _write_pmc(d, seq, counter, values):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value",
                    "Start_Timestamp", "End_Timestamp"])
        for i, (n, v) in enumerate(zip(seq, values), 1):
            w.writerow([i, 1024, n, counter, v, 0, 1000])


def test_phases_by_dispatch_order(tmp_path):
    _write_trace(str(tmp_path / "t"), SEQ)
    ph = ps.phases(ps.read_trace(str(tmp_path / "t")))
    assert [d["id"] for d in ph["hot"]] == [2, 3, 4, 5, 6, 7]
    assert [d["id"] for d in ph["cold"]] == [9, 11, 12]
    assert [d["id"] for d in ph["variants"]] == [16, 17, 18, 19, 20]
    # trace durations: dispatch i lasts i microseconds
    assert [d["us"] for d in ph["hot"]] == [2.0, 3.0, 4.0, 5.0, 6.0, 7.0]


def test_counters_json_scales_by_the_copy(tmp_path, monkeypatch):
    """FETCH_SIZE / WRITE_SIZE of the steady-state kernels are averaged, the
    scale is what the counters read for the 1 GiB copy, and counters.json is
    keyed to the kernel source."""
    _write_trace(str(tmp_path / "t"), SEQ)
    fetch = [0, 10, 20, 1, 30, 40, 3, 0, 99, 0, 99, 99, 0, 524288, 524288, 7, 7, 0, 1, 7]
    write = [0, 5, 6, 1, 7, 8, 1, 0, 99, 0, 99, 99, 0, 1048576, 1048576, 7, 7, 0, 1, 7]
    _write_pmc(str(tmp_path / "p1"), SEQ, "FETCH_SIZE", fetch)
    _write_pmc(str(tmp_path / "p2"), SEQ, "WRITE_SIZE", write)
    cmds = tmp_path / "cmds.txt"
    cmds.write_text("rocprofv3 ... -- python3 bench.py\n")
    out = tmp_path / "q.md"
    cj = tmp_path / "counters.json"
    ps.main(["--workload", "qwen05", "--trace", str(tmp_path / "t"), "--pmc", str(tmp_path / "p1"),
             str(tmp_path / "p2"), "--commands", str(cmds), "--out", str(out),
             "--counters-json", str(cj)])
    c = json.loads(cj.read_text())
    assert c["kernel_source_sha256_16"] == ps.kernel_hash()
    assert c["copy_calibration"]["fetch_scale"] == 2.0 and c["copy_calibration"]["write_scale"] == 1.0
    e = c["workloads"]["qwen05"]
    assert e["fwd"] == {"fetch_kib": 20.0, "write_kib": 6.0}      # mean of 10, 30 and 5, 7
    assert e["bwd"] == {"fetch_kib": 30.0, "write_kib": 7.0}
    assert e["finalize"] == {"fetch_kib": 2.0, "write_kib": 1.0}
    text = out.read_text()
    assert "rocprofv3 ... -- python3 bench.py" in text and ps.kernel_hash() in text

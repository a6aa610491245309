#!/usr/bin/env python3
"""Summaries of rocprofv3 output for profiles/: kernel durations from a
`--kernel-trace --stats` run of bench.py and per-dispatch counters from
`--pmc` runs of the same command, as a markdown report per workload and the
HBM-traffic figures bench.py reads (profiles/counters.json).

    python profile_summary.py --workload qwen05 --trace DIR --pmc DIR [DIR ...] \
        --commands FILE --out profiles/qknr_qwen05_trace_and_counters.md [--counters-json PATH]

DIR is a rocprofv3 output directory (`-d DIR -o run -f csv`).  FILE holds the
commands that produced the directories, copied into the report verbatim.

Phases of a bench.py run, told apart by dispatch order: the steady-state calls
(clock settling, warmup, timed steps, per-call loops) come before the first
cache-flush kernel; each call that directly follows a flush is a cold call; the
bandwidth probes (copy and two-read/one-write kernels) follow; the extended
entry points (HIP-graph replays) come after the last probe.

HBM bytes: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what the
same counters read for the bench's 1 GiB copy (1048576 KiB read and written).
The raw requests explain the scale: on this part FETCH_SIZE is
(TCC_BUBBLE * 128 + (TCC_EA0_RDREQ - TCC_BUBBLE - TCC_EA0_RDREQ_32B) * 64 +
TCC_EA0_RDREQ_32B * 32) / 1024, which prices every read request that is neither
32 B nor a "bubble" at 64 B, while the streaming kernels' read requests are
128 B each (RDREQ * 128 B matches the bytes read); writes are 64-B requests
(TCC_EA0_WRREQ_64B), which WRITE_SIZE prices right.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

KERNEL_SRC = os.path.join(ROOT, "qk_norm_rope_amd", "csrc", "qknr.hip")
COPY_KIB = 1048576.0  # the bench's 1 GiB copy
FLUSH, COPY, STREAM2, EMPTY = "bench_flush", "bench_copy", "bench_stream2", "bench_empty"


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def _args(name: str) -> list[str]:
    m = re.search(r"<(.*)>\(", name)
    if not m:
        return []
    return [a.strip() for a in m.group(1).split(",")]


def friendly(name: str) -> str | None:
    """A short name for this library's kernels; None for others."""
    io = lambda a: "bf16" if "Bf16" in a else "fp32"  # noqa: E731
    if "bench_flush_kernel" in name:
        return FLUSH
    if "bench_copy_kernel" in name:
        return COPY
    if "bench_stream2_kernel" in name:
        return STREAM2
    if "bench_empty_kernel" in name:
        return EMPTY
    if "qknr_dw_finalize_kernel" in name:
        return "qknr_dw_finalize_kernel"
    if "qknr_group_finalize_kernel" in name:
        return "qknr_group_finalize_kernel"
    if "qknr_bfd_emit_kernel" in name:
        return "qknr_bfd_emit_kernel"
    a = _args(name)
    if "qknr_bfd_place_kernel" in name:
        return "qknr_bfd_place_kernel<%s>" % ", ".join(a)
    if "qknr_kernel<" in name and len(a) == 7:
        tags = [io(a[0]), "D=%s" % a[1], "bwd" if a[3] == "true" else "fwd"]
        for flag, tag in ((a[4], "interleaved"), (a[5], "slot-mapped K"), (a[6], "options")):
            if flag == "true":
                tags.append(tag)
        return "qknr_kernel<%s>" % ", ".join(tags)
    for k in ("qknr_gwave_kernel", "qknr_group_kernel"):
        if k + "<" in name and len(a) == 5:
            tags = [io(a[0]), "D=%s" % a[1], "bwd" if a[2] == "true" else "fwd"]
            for flag, tag in ((a[3], "interleaved"), (a[4], "slot-mapped K")):
                if flag == "true":
                    tags.append(tag)
            return "%s<%s>" % (k, ", ".join(tags))
    return None


def read_trace(d: str) -> list[dict]:
    out = []
    with open(os.path.join(d, "run_kernel_trace.csv")) as fh:
        for r in csv.DictReader(fh):
            out.append({"id": int(r["Dispatch_Id"]), "name": friendly(r["Kernel_Name"]),
                        "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3,
                        "grid": int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]),
                        "wg": int(r["Workgroup_Size_X"]), "lds": int(r["LDS_Block_Size"])})
    out.sort(key=lambda x: x["id"])
    return out


def read_pmc(d: str) -> list[dict]:
    per = {}
    with open(os.path.join(d, "run_counter_collection.csv")) as fh:
        for r in csv.DictReader(fh):
            i = int(r["Dispatch_Id"])
            e = per.setdefault(i, {"id": i, "name": friendly(r["Kernel_Name"]),
                                   "grid": int(r["Grid_Size"]), "c": {},
                                   "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3})
            e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [per[i] for i in sorted(per)]


def phases(disp: list[dict]) -> dict:
    """Split this library's dispatches into steady-state (hot), cold (directly
    after a flush) and variants (after the run of bandwidth probes that
    follows the cold calls; the variants' own probes, an empty kernel and
    small copies beside the decode steps, are listed with them)."""
    names = [d["name"] for d in disp]
    first_flush = next((i for i, n in enumerate(names) if n == FLUSH), len(disp))
    probes = [i for i, n in enumerate(names) if n in (COPY, STREAM2)]
    last_probe = len(disp)
    if probes:
        last_probe = probes[0]
        while last_probe + 1 < len(disp) and names[last_probe + 1] in (COPY, STREAM2, FLUSH, None):
            last_probe += 1
    hot, cold, var = [], [], []
    prev = None
    for i, d in enumerate(disp):
        n = d["name"]
        if i > last_probe and n in (COPY, EMPTY):
            var.append(d)
            prev = n
            continue
        if n is None or n in (FLUSH, COPY, STREAM2, EMPTY):
            prev = n
            continue
        if i < first_flush:
            hot.append(d)
        elif i > last_probe:
            var.append(d)
        elif prev == FLUSH or (cold and cold[-1]["name"] != n and names[i - 1] == cold[-1]["name"]):
            # a cold call and the small kernel that ends it (the dw finalize)
            cold.append(d)
        prev = n
    return {"hot": hot, "cold": cold, "variants": var}


def _pct(v: list[float], f: float) -> float:
    s = sorted(v)
    return s[min(len(s) - 1, int(f * len(s)))]


def duration_table(disp: list[dict], group_grid: bool = False) -> list[str]:
    groups: dict = {}
    for d in disp:
        key = (d["name"], d["grid"]) if group_grid else d["name"]
        groups.setdefault(key, []).append(d)
    rows = ["| kernel | calls | avg us | median us | p10 us | p90 us | min us | grid threads | workgroup |"
            " LDS bytes |", "|---|---|---|---|---|---|---|---|---|---|"]
    for key, ds in groups.items():
        us = [d["us"] for d in ds]
        name = key[0] if group_grid else key
        rows.append("| %s | %d | %.2f | %.2f | %.2f | %.2f | %.2f | %d | %d | %d |" % (
            name, len(us), statistics.mean(us), statistics.median(us), _pct(us, 0.1), _pct(us, 0.9),
            min(us), ds[0]["grid"], ds[0].get("wg", 0), ds[0].get("lds", 0)))
    return rows


def counters_by_kernel(runs: list[list[dict]]) -> tuple[dict, dict]:
    """Mean counter value per steady-state dispatch of each kernel, over every
    pmc run; and the 1 GiB copies' FETCH_SIZE / WRITE_SIZE."""
    acc: dict = {}
    cal = {"FETCH_SIZE": [], "WRITE_SIZE": []}
    for disp in runs:
        for d in phases(disp)["hot"]:
            for c, v in d["c"].items():
                acc.setdefault(d["name"], {}).setdefault(c, []).append(v)
        for d in disp:
            if d["name"] == COPY:
                for c in cal:
                    if c in d["c"]:
                        cal[c].append(d["c"][c])
    mean = {k: {c: statistics.mean(v) for c, v in cs.items()} for k, cs in acc.items()}
    # the 1 GiB copies are the largest copies of the run
    calib = {}
    for c, v in cal.items():
        if v:
            big = [x for x in v if x > 0.4 * max(v)]
            calib[c] = statistics.mean(big)
    return mean, calib


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--trace", required=True)
    ap.add_argument("--pmc", nargs="*", default=[])
    ap.add_argument("--commands", required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--counters-json", default=os.path.join(ROOT, "profiles", "counters.json"))
    a = ap.parse_args(argv)

    from workloads import configs

    w = configs.get(a.workload)
    trace = read_trace(a.trace)
    ph = phases(trace)
    runs = [read_pmc(d) for d in a.pmc]
    cm, calib = counters_by_kernel(runs)
    fs = COPY_KIB / calib["FETCH_SIZE"] if "FETCH_SIZE" in calib else None
    ws = COPY_KIB / calib["WRITE_SIZE"] if "WRITE_SIZE" in calib else None
    io = "bf16" if w.dtype == "bf16" else "fp32"
    main_f = "qknr_kernel<%s, D=%d, fwd>" % (io, w.head_dim)
    main_b = "qknr_kernel<%s, D=%d, bwd>" % (io, w.head_dim)
    fin = "qknr_dw_finalize_kernel"
    with open(a.commands) as fh:
        commands = fh.read().strip()

    L = ["# Kernel trace and counters: %s" % w.description, "",
         "Produced on one MI355X (gfx950) from the repository root by these commands (rocprofv3 runs "
         "from /tmp with `TMPDIR=/tmp`, paths absolute), then this report by `profile_summary.py`:", "",
         "```", commands, "```", "",
         "Kernel source sha256 (first 16 hex): `%s`." % kernel_hash(), "",
         "## Dense path: kernel durations (rocprofv3 --kernel-trace)", "",
         "Steady-state dispatches: clock settling, warmup, the timed steps and the per-call loops "
         "(everything before the first cache flush).", ""]
    L += duration_table(ph["hot"])
    L += ["", "Each call alone and cold (the bench's `cold_fwd` / `cold_bwd`: a 1 GiB flush kernel before "
               "every call, outside the call's events):", ""]
    L += duration_table(ph["cold"])
    hot = {}
    for d in ph["hot"]:
        hot.setdefault(d["name"], []).append(d["us"])
    if main_b in hot and fin in hot:
        tb = statistics.mean(hot[main_b]) + statistics.mean(hot[fin])
        tf = statistics.mean(hot[main_f])
        L += ["", "From the trace: forward %.2f us per call = %.1f GB/s of algorithmic bytes (%.3f of 8 TB/s); "
                  "backward call (main kernel + dw finalize) %.2f + %.2f = %.2f us = %.1f GB/s (%.3f of "
                  "8 TB/s)." % (tf, w.fwd_bytes() / tf / 1e3, w.fwd_bytes() / tf / 8e6,
                                statistics.mean(hot[main_b]), statistics.mean(hot[fin]), tb,
                                w.bwd_bytes() / tb / 1e3, w.bwd_bytes() / tb / 8e6)]
        tm = statistics.mean(hot[main_b])
        empty = [d["us"] for d in ph["variants"] if d["name"] == EMPTY]
        L += ["", "The backward's main kernel alone moves the backward's algorithmic bytes at %.1f GB/s (%.3f of "
                  "8 TB/s). The bench times the whole backward call with HIP events and no profiler, so its "
                  "`roofline.achieved` lies between these two figures: the finalize sums a few hundred KB of "
                  "partials, and most of its traced duration is the profiler's own per-dispatch cost%s."
              % (w.bwd_bytes() / tm / 1e3, w.bwd_bytes() / tm / 8e6,
                 " (an empty kernel reads %.2f us in the same trace)" % statistics.mean(empty) if empty else "")]
    if ph["variants"]:
        L += ["", "## Extended entry points: kernel durations (HIP-graph replays)", "",
              "After the bandwidth probes: the dense calls and Q/K as views of a fused QKV buffer rewritten "
              "in place (same kernels), interleaved pairs, QK-LayerNorm with biases and a frequency table "
              "(`options`), norm groups with [H, D] weights (the wave kernel), decode steps writing K "
              "through a slot map (B = 1, 64, 256 tokens: the grid tells them apart) and the device BFD "
              "packer; one row per kernel and grid size.", ""]
        L += duration_table(ph["variants"], group_grid=True)
    entry = {}
    if runs:
        L += ["", "## HBM traffic per dispatch (rocprofv3 --pmc)", ""]
        if fs and ws:
            L += ["Calibration with the bench's 1 GiB copy (1048576 KiB read, 1048576 KiB written): "
                  "FETCH_SIZE reads %.0f KiB (scale %.4f), WRITE_SIZE %.0f KiB (scale %.4f)."
                  % (calib["FETCH_SIZE"], fs, calib["WRITE_SIZE"], ws), ""]
        L += ["| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled HBM bytes | algorithmic bytes | ratio |",
              "|---|---|---|---|---|---|"]
        for k, alg in ((main_f, w.fwd_bytes()), (main_b, w.bwd_bytes()), (fin, None)):
            c = cm.get(k, {})
            if "FETCH_SIZE" in c and "WRITE_SIZE" in c and fs and ws:
                byts = (c["FETCH_SIZE"] * fs + c["WRITE_SIZE"] * ws) * 1024.0
                L.append("| %s | %.1f | %.1f | %.0f | %s | %s |" % (
                    k, c["FETCH_SIZE"], c["WRITE_SIZE"], byts, alg if alg else "-",
                    "%.3f" % (byts / alg) if alg else "-"))
                part = {"qknr_kernel<%s, D=%d, fwd>" % (io, w.head_dim): "fwd",
                        main_b: "bwd", fin: "finalize"}[k]
                entry[part] = {"fetch_kib": c["FETCH_SIZE"], "write_kib": c["WRITE_SIZE"]}
        raw = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_BUBBLE_sum", "TCC_EA0_WRREQ_sum",
               "TCC_EA0_WRREQ_64B_sum")
        if any(r in cm.get(main_b, {}) for r in raw):
            L += ["", "Raw L2-to-memory requests per dispatch (the explanation of the FETCH_SIZE scale: "
                      "read requests are 128 B, which the FETCH_SIZE formula prices at 64 B):", "",
                  "| kernel | RDREQ | RDREQ_32B | BUBBLE | RDREQ x 128 B | FETCH_SIZE formula x 1024 B |"
                  " WRREQ | WRREQ_64B | WRREQ_64B x 64 B |", "|---|---|---|---|---|---|---|---|---|"]
            for k in (main_f, main_b, COPY):
                c = cm.get(k, {})
                src = c
                if k == COPY:
                    # steady-state copies are not in the hot phase; take the 1 GiB ones
                    big = [d["c"] for disp in runs for d in disp
                           if d["name"] == COPY and "TCC_EA0_RDREQ_sum" in d["c"]]
                    if not big:
                        continue
                    mx = max(b["TCC_EA0_RDREQ_sum"] for b in big)
                    sel = [b for b in big if b["TCC_EA0_RDREQ_sum"] > 0.4 * mx]
                    src = {n: statistics.mean(b[n] for b in sel) for n in sel[0]}
                    big64 = [d["c"]["TCC_EA0_WRREQ_64B_sum"] for disp in runs for d in disp
                             if d["name"] == COPY and "TCC_EA0_WRREQ_64B_sum" in d["c"]]
                    if big64:
                        m64 = max(big64)
                        src["TCC_EA0_WRREQ_64B_sum"] = statistics.mean(x for x in big64 if x > 0.4 * m64)
                    k = "bench copy, 1 GiB"
                rd, r32, bub = (src.get(n, float("nan")) for n in raw[:3])
                wr, w64 = src.get(raw[3], float("nan")), src.get(raw[4], float("nan"))
                fetch_formula = bub * 128 + (rd - bub - r32) * 64 + r32 * 32
                L.append("| %s | %.0f | %.0f | %.0f | %.0f | %.0f | %.0f | %.0f | %.0f |" % (
                    k, rd, r32, bub, rd * 128, fetch_formula, wr, w64, w64 * 64))
        sq = ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD",
              "SQ_INSTS_VMEM_WR", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU",
              "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_LDS", "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE")
        ks = [k for k in (main_f, main_b, fin) if "SQ_WAVES" in cm.get(k, {})]
        if ks:
            L += ["", "## SQ counters per dispatch (rocprofv3 --pmc; totals over the device, per wave where "
                      "divided by SQ_WAVES)", "",
                  "| kernel | " + " | ".join(sq) + " | VALU / wave | SALU / wave | LDS / wave | VALUBusy % |",
                  "|---|" + "---|" * (len(sq) + 4)]
            for k in ks:
                c = cm[k]
                waves = c.get("SQ_WAVES", float("nan"))
                grbm = c.get("GRBM_GUI_ACTIVE", float("nan"))
                # VALUBusy as rocprof derives it: active VALU cycles (x4 per
                # instruction issue) over the SIMDs' busy cycles; GRBM_GUI_ACTIVE
                # is summed over the 8 XCDs here, hence per XCD / 8
                simds = 256 * 4
                busy = 100.0 * c.get("SQ_ACTIVE_INST_VALU", float("nan")) * 4 / simds / (grbm / 8)
                L.append("| %s | " % k + " | ".join("%.0f" % c.get(n, float("nan")) for n in sq)
                         + " | %.0f | %.0f | %.0f | %.1f |" % (
                             c.get("SQ_INSTS_VALU", float("nan")) / waves,
                             c.get("SQ_INSTS_SALU", float("nan")) / waves,
                             c.get("SQ_INSTS_LDS", float("nan")) / waves, busy))
            L += ["", "GRBM_GUI_ACTIVE over the kernel's trace duration gives the cycle count of the 8 XCDs "
                      "together; VALUBusy above takes one XCD's share (/ 8)."]
    # the bench line printed by the traced run itself
    log = os.path.join(os.path.dirname(a.trace.rstrip("/")), os.path.basename(a.trace.rstrip("/")) + ".log")
    if os.path.exists(log):
        with open(log) as fh:
            lines = [x for x in fh if x.startswith("{")]
        if lines:
            L += ["", "## Bench line printed by the traced command", "", "```", lines[-1].strip(), "```"]
    with open(a.out, "w") as fh:
        fh.write("\n".join(L) + "\n")
    if entry and fs and ws:
        try:
            with open(a.counters_json) as fh:
                cj = json.load(fh)
        except (OSError, ValueError):
            cj = {}
        if cj.get("kernel_source_sha256_16") != kernel_hash():
            cj = {"kernel_source_sha256_16": kernel_hash(), "workloads": {}}
        cj["copy_calibration"] = {"fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
                                  "copy_fetch_kib": calib["FETCH_SIZE"],
                                  "copy_write_kib": calib["WRITE_SIZE"], "copy_bytes": 1 << 30}
        cj.setdefault("workloads", {})[a.workload] = entry
        with open(a.counters_json, "w") as fh:
            json.dump(cj, fh, indent=1)
    print("wrote", a.out)


if __name__ == "__main__":
    main()

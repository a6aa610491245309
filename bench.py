#!/usr/bin/env python3
"""Benchmark of the fused QK-Norm + RoPE forward + backward on one MI355X.

A step is one forward and one backward (the whole hot path) over one batch of
the chosen workload; the default workload is the Qwen2.5-0.5B-shaped one
(8 x 4096 tokens, 14 Q / 2 KV heads, head_dim 64, bf16 storage, fp32
arithmetic), and the 7B-shaped workload (4 x 8192 tokens, 32 Q / 8 KV heads,
head_dim 128) is measured the same way in the same run.  Inputs are resident
in HBM before timing starts.  Several complete input/output sets are rotated
so that the bytes touched between two uses of a set exceed the 256 MB
Infinity Cache.

Timing protocol, per workload:
  1. clock settling: untimed forward + backward steps for at least 50 ms of GPU
     time (the GPU needs about 30 ms of work to reach steady clocks), reported
     as `clock_settle`;
  2. exactly --warmup untimed steps;
  3. exactly --steps timed steps between two HIP events on the launch stream,
     with a synchronisation on each side; step i runs the forward of set i and
     the backward of set i - 1, so the backward never reads what the forward
     just read;
  4. per-call durations: --steps back-to-back launches of each call alone
     (rotating sets) between two events; the roofline reports the dominant
     call, the backward (its main kernel plus the small dw finalize kernel).

Prints one JSON line.  A "variants" object times the extended entry points on
the default shape as HIP-graph replays; "cpu_baseline" times the fp64 oracle on
the host cores and reports the parity statistics of the GPU outputs against it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload qwen05|packed|7b|long|tiny]
                    [--second 7b|none] [--no-cpu-baseline] [--no-variants]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QK-Norm+RoPE fwd+bwd tokens/s and achieved HBM GB/s (% of peak), 1 GPU"
HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, AMD public specification
MALL_BYTES = 256 << 20      # Infinity Cache
SETTLE_MS = 50.0            # GPU time of untimed work before the warmup steps
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
KERNEL_SRC = os.path.join(ROOT, "qk_norm_rope_amd", "csrc", "qknr.hip")


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen05")
    ap.add_argument("--second", default="7b",
                    help="a second workload measured the same way, or 'none'")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="approximate CPU time of the oracle's multi-thread runs")
    ap.add_argument("--cold-reps", type=int, default=100,
                    help="repetitions of each call timed alone after a cache flush")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="GPU milliseconds of untimed steps before the warmup (profiler runs "
                         "shorten it)")
    return ap.parse_args(argv)


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def traffic_from_counters(name: str):
    """HBM bytes of one backward call (main kernel + dw finalize) from the
    committed rocprofv3 --pmc readings in profiles/counters.json: FETCH_SIZE and
    WRITE_SIZE in KiB per dispatch, each scaled by what the same counter reads
    for a copy of known size.  None when the file holds no readings for the
    current kernel source (the counters cannot be read from inside this
    process; they come from separate rocprofv3 runs of this script)."""
    try:
        with open(COUNTERS) as fh:
            c = json.load(fh)
    except (OSError, ValueError):
        return None
    e = c.get("workloads", {}).get(name)
    if not e or c.get("kernel_source_sha256_16") != kernel_hash():
        return None
    scale_f = c["copy_calibration"]["fetch_scale"]
    scale_w = c["copy_calibration"]["write_scale"]
    total = 0.0
    for part in ("bwd", "finalize"):   # the two launches of one backward call
        k = e.get(part)
        if not k:
            return None
        total += (k["fetch_kib"] * scale_f + k["write_kib"] * scale_w) * 1024.0
    return total


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _median_time(fn, reps=None, budget_s=None, cores=1):
    """Median wall time of fn() over reps calls (at least 3), or over as many
    as fit budget_s CPU-seconds at `cores` threads."""
    ts = []
    t_all = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
        if reps is not None and len(ts) >= reps:
            break
        if budget_s is not None and len(ts) >= 3 and (time.perf_counter() - t_all) * cores >= budget_s:
            break
        if len(ts) >= 200:
            break
    return statistics.median(ts), len(ts)


def cpu_baseline(w, budget_s: float, gpu_out=None):
    """The oracle, as it stands (fp64 C, scalar loops), on the host cores: the
    whole workload's forward and backward timed separately at every core the
    process may use (median over repetitions), one thread on the tiny workload
    and on the first 1024 tokens of this one, and the oracle's BFD packer on
    the benchmark's two document mixes.  With gpu_out (host copies of the GPU's
    outputs for set 0) also the parity statistics of the GPU against the
    oracle on every element."""
    import numpy as np

    import oracle
    from oracle import parity
    from workloads import bfd as host_bfd, configs, gen

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    inp = gen.make_inputs(w, backward=w.backward)
    dec = lambda a: oracle.decode(a, w.dtype)  # noqa: E731
    q, k, wq, wk = dec(inp["q"]), dec(inp["k"]), dec(inp["wq"]), dec(inp["wk"])
    dyq, dyk = (dec(inp["dyq"]), dec(inp["dyk"])) if w.backward else (None, None)
    args = (w.rotary_dim, w.eps, w.theta)
    out = {}
    t_f, n_f = _median_time(lambda: out.__setitem__("y", oracle.fwd(q, k, wq, wk, inp["pos"], *args,
                                                                       threads=cores)),
                            budget_s=budget_s * (0.4 if w.backward else 1.0), cores=cores)
    res = {"unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu_model": cpu_model(),
           "fwd": {"ms": round(t_f * 1e3, 3), "tokens_per_s": round(w.tokens / t_f, 1),
                   "GBps_equiv": round(w.fwd_bytes() / t_f / 1e9, 3)}}
    if w.backward:
        t_b, n_b = _median_time(lambda: out.__setitem__("g", oracle.bwd(q, k, wq, wk, inp["pos"], dyq,
                                                                           dyk, *args, threads=cores)),
                                budget_s=budget_s * 0.6, cores=cores)
        res["bwd"] = {"ms": round(t_b * 1e3, 3), "tokens_per_s": round(w.tokens / t_b, 1),
                      "GBps_equiv": round(w.bwd_bytes() / t_b / 1e9, 3)}
        res["value"] = w.tokens / (t_f + t_b)
        res["GBps_equiv"] = round((w.fwd_bytes() + w.bwd_bytes()) / (t_f + t_b) / 1e9, 3)
        res["sample"] = ("%s: the whole workload (%d tokens), fwd median of %d runs, bwd median of %d "
                         "runs, fp64 C oracle on %d threads (static token ranges)"
                         % (w.name, w.tokens, n_f, n_b, cores))
    else:
        res["value"] = w.tokens / t_f
        res["GBps_equiv"] = res["fwd"]["GBps_equiv"]
        res["sample"] = ("%s: the whole workload (%d tokens, forward only), median of %d runs, fp64 C "
                         "oracle on %d threads (static token ranges)" % (w.name, w.tokens, n_f, cores))
    # one thread: the tiny workload whole, and the first 1024 tokens of this one
    single = {}
    for name, ww, n1 in (("tiny", configs.TINY, configs.TINY.tokens), (w.name, w, min(w.tokens, 1024))):
        ii = gen.make_inputs(ww, 0, n1, backward=ww.backward)
        d1 = lambda a: oracle.decode(a, ww.dtype)  # noqa: E731,B023
        qq, kk, wwq, wwk = d1(ii["q"]), d1(ii["k"]), d1(ii["wq"]), d1(ii["wk"])
        gq, gk = (d1(ii["dyq"]), d1(ii["dyk"])) if ww.backward else (None, None)
        a1 = (ww.rotary_dim, ww.eps, ww.theta)
        tf, _ = _median_time(lambda: oracle.fwd(qq, kk, wwq, wwk, ii["pos"], *a1, threads=1), reps=3)
        single[name] = {"tokens": n1, "fwd_tokens_per_s": round(n1 / tf, 1)}
        if ww.backward:
            tb, _ = _median_time(lambda: oracle.bwd(qq, kk, wwq, wwk, ii["pos"], gq, gk, *a1,
                                                    threads=1), reps=3)
            single[name].update(bwd_tokens_per_s=round(n1 / tb, 1),
                                fwd_bwd_tokens_per_s=round(n1 / (tf + tb), 1))
    res["single_thread"] = single
    # the oracle's Best-Fit-Decreasing packer on the benchmark's two mixes
    pw = configs.get("packed")
    docs = host_bfd.draw_lengths(gen.rng(pw.seed, gen.S_DOCS), pw.doc_len_min, pw.doc_len_max,
                                 pool_tokens=8 * pw.tokens)
    big = np.clip(np.rint(np.exp(np.random.default_rng(5).uniform(np.log(16), np.log(4096), 4000))),
                  16, 4096).astype(np.int32)
    packs = {}
    for name, lengths, cap, max_bins in (("packed_workload_docs", np.asarray(docs, np.int32), pw.tokens, 64),
                                         ("4000_docs_into_4096", big, 4096, 2048)):
        t, n = _median_time(lambda: oracle.bfd_pack(lengths, cap, max_bins), reps=5)
        r = oracle.bfd_pack(lengths, cap, max_bins)
        packs[name] = {"us": round(t * 1e6, 2), "docs": int(len(lengths)), "runs": n,
                       "bins": int(r.get("bins", -1)), "status": int(r["status"])}
    res["bfd_pack"] = packs
    if gpu_out is not None:
        y = out["y"]
        ref = {"yq": y[0], "yk": y[1]}
        if w.backward:
            g = out["g"]
            ref.update(dq=g[0], dk=g[1], dwq=g[2], dwk=g[3])
        par = {}
        for key, o in ref.items():
            try:
                st = parity.compare(oracle.decode(gpu_out[key], w.dtype), o, w.dtype, key,
                                    row_sum=key.startswith("dw"))
                par[key] = parity.brief(st)
            except AssertionError as e:
                par[key] = {"fail": str(e)[:300]}
        res["parity"] = dict(par, rule="bf16: 2 ulp of the oracle's rounded value with a 2^-16 "
                                       "row-RMS floor; beyond_strict_2ulp counts elements past "
                                       "a strict 2 ulp" if w.dtype == "bf16" else "fp32: 2e-5")
    return res


def graph_time(calls, reps, stream):
    """Capture the launches of `calls` (in order) into one HIP graph, replay it
    `reps` times between two events, and return microseconds per call.  This
    measures the kernels back to back without the Python binding's per-call
    host time, which exceeds a short kernel's duration (decode)."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(reps):
        g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / (reps * len(calls))
    del g
    return us


def measure_variants(qk, w, base, sets, k, stream):
    """Per-call times of the extended entry points, each as HIP-graph replays of
    back-to-back calls over the rotated sets (see graph_time), next to the
    dense calls timed the same way.  Fused: Q and K are views of a
    [T, (hq + 2 hkv) D] buffer (and the upstream gradients of another), the
    forward rewrites them in place and the backward writes dq/dk over the
    gradient buffer; algorithmic bytes are the dense ones (V is not touched).
    Interleaved: dense tensors, pairs (2i, 2i+1).  LayerNorm + biases + table:
    the norm variant with every option of qknr_fwd_opt / qknr_bwd_opt.  Groups:
    norm groups (GQA-sized for q, layerwise for k) with [H, D] weights (the
    wave kernel when every group lies within one wave stage, else the
    whole-token kernel).  BFD: the device packer.  Decode: one token per
    sequence at positions up to 256k, Q dense, K written through a slot map
    into a paged cache [slots, hkv, D]; latency-bound (a launch floor, measured
    beside them as decode_floor, plus one memory round trip); also with the
    groups row's norm groups and [H, D] weights."""
    import numpy as np
    import torch

    dev = base["q"].device
    T, hq, hkv, D = w.tokens, w.hq, w.hkv, w.head_dim
    dt = base["q"].dtype
    args = (w.rotary_dim, w.eps, w.theta)
    width = (hq + 2 * hkv) * D
    nsets = len(sets)
    ncalls = 4 * nsets
    reps = max(2, k // ncalls)
    ws = torch.zeros(max(16, qk.qknr_bwd_workspace_bytes(T, hq, hkv, D, dt)), dtype=torch.uint8,
                     device=dev)
    dwq, dwk = torch.empty_like(base["wq"]), torch.empty_like(base["wk"])

    def rates(f_us, b_us):
        return {"fwd_us": round(f_us, 3), "fwd_alg_GBps": round(w.fwd_bytes() / f_us / 1e3, 1),
                "bwd_us": round(b_us, 3), "bwd_alg_GBps": round(w.bwd_bytes() / b_us / 1e3, 1)}

    def timed_pair(fwd_i, bwd_i):
        f = graph_time([lambda i=i: fwd_i(i % nsets) for i in range(ncalls)], reps, stream)
        b = graph_time([lambda i=i: bwd_i(i % nsets) for i in range(ncalls)], reps, stream)
        return rates(f, b)

    out = {"timing": "HIP graph of %d back-to-back calls over %d rotated sets, replayed %d times"
                     % (ncalls, nsets, reps)}

    # dense, for reference
    def dfwd(i):
        s = sets[i]
        qk.qknr_fwd(s["q"], s["k"], s["wq"], s["wk"], s["pos"], *args, q_out=s["yq"], k_out=s["yk"])

    def dbwd(i):
        s = sets[i]
        qk.qknr_bwd(s["q"], s["k"], s["wq"], s["wk"], s["pos"], s["dyq"], s["dyk"], *args,
                    dq=s["dq"], dk=s["dk"], dwq=s["dwq"], dwk=s["dwk"], workspace=ws)

    out["dense"] = timed_pair(dfwd, dbwd)

    # fused QKV views, in place
    view = lambda b, o, h: b[:, o: o + h * D].unflatten(1, (h, D))  # noqa: E731
    fused = []
    for i in range(nsets):
        x = torch.empty(T, width, dtype=dt, device=dev)
        x[:, : hq * D] = base["q"].reshape(T, -1)
        x[:, hq * D: (hq + hkv) * D] = base["k"].reshape(T, -1)
        g = torch.empty(T, width, dtype=dt, device=dev)
        g[:, : hq * D] = base["dyq"].reshape(T, -1)
        g[:, hq * D: (hq + hkv) * D] = base["dyk"].reshape(T, -1)
        fused.append((x, g, view(x, 0, hq), view(x, hq * D, hkv), view(g, 0, hq),
                      view(g, hq * D, hkv)))

    def ffwd(i):
        _, _, q, kk, _, _ = fused[i]
        qk.qknr_fwd_ex(q, kk, base["wq"], base["wk"], base["pos"], *args, q_out=q, k_out=kk)

    def fbwd(i):
        _, _, q, kk, gq, gk = fused[i]
        qk.qknr_bwd_ex(q, kk, base["wq"], base["wk"], base["pos"], gq, gk, *args, dq=gq, dk=gk,
                       dwq=dwq, dwk=dwk, workspace=ws)

    out["fused_qkv_in_place"] = dict(timed_pair(ffwd, fbwd), token_stride=width)
    del fused

    # interleaved pairs, dense tensors
    def ifwd(i):
        s = sets[i]
        qk.qknr_fwd_ex(s["q"], s["k"], s["wq"], s["wk"], s["pos"], *args,
                       flags=qk.QKNR_FLAG_INTERLEAVED, q_out=s["yq"], k_out=s["yk"])

    def ibwd(i):
        s = sets[i]
        qk.qknr_bwd_ex(s["q"], s["k"], s["wq"], s["wk"], s["pos"], s["dyq"], s["dyk"], *args,
                       flags=qk.QKNR_FLAG_INTERLEAVED, dq=s["dq"], dk=s["dk"], dwq=s["dwq"],
                       dwk=s["dwk"], workspace=ws)

    out["interleaved"] = timed_pair(ifwd, ibwd)

    # QK-LayerNorm with [D] biases, a caller frequency table (position
    # interpolation by 4 on every pair) and an attention factor; the backward
    # also writes the bias gradients.  Bias bytes (2 D elements) are left out
    # of the algorithmic bytes, like the weights.
    bq, bk = torch.zeros_like(base["wq"]), torch.zeros_like(base["wk"])
    dbq, dbk = torch.empty_like(bq), torch.empty_like(bk)
    h = w.rotary_dim // 2
    table = [w.theta ** (-2.0 * i / w.rotary_dim) / 4.0 for i in range(h)]
    opt = dict(flags=qk.QKNR_FLAG_LAYERNORM, inv_freq=table, attention_factor=1.1)

    def lfwd(i):
        s = sets[i]
        qk.qknr_fwd_opt(s["q"], s["k"], s["wq"], s["wk"], s["pos"], *args, bq=bq, bk=bk,
                        q_out=s["yq"], k_out=s["yk"], **opt)

    def lbwd(i):
        s = sets[i]
        qk.qknr_bwd_opt(s["q"], s["k"], s["wq"], s["wk"], s["pos"], s["dyq"], s["dyk"], *args,
                        bias_grads=True, dq=s["dq"], dk=s["dk"], dwq=s["dwq"], dwk=s["dwk"],
                        dbq=dbq, dbk=dbk, workspace=ws, **opt)

    out["layernorm_bias_table"] = timed_pair(lfwd, lbwd)

    # Norm groups and per-head weights (the norm-group kernels): q heads in
    # GQA-sized groups (hq / hkv heads share one inverse RMS), k normed over
    # all its heads (layerwise), [H, D] weights and biases; the backward writes
    # [H, D] weight and bias gradients.
    gq = hq // hkv
    hwq = torch.ones(hq, D, dtype=dt, device=dev)
    hwk = torch.ones(hkv, D, dtype=dt, device=dev)
    hbq, hbk = torch.zeros_like(hwq), torch.zeros_like(hwk)
    hg = [torch.empty_like(hwq), torch.empty_like(hwk), torch.empty_like(hwq), torch.empty_like(hwk)]
    gopt = dict(flags=qk.QKNR_FLAG_HEAD_WEIGHTS, norm_groups=(gq, hkv))
    gws = torch.zeros(max(16, qk.qknr_bwd_opt_workspace_bytes(T, hq, hkv, D, w.rotary_dim, dt,
                                                              **gopt)), dtype=torch.uint8,
                      device=dev)

    def gfwd(i):
        s = sets[i]
        qk.qknr_fwd_opt(s["q"], s["k"], hwq, hwk, s["pos"], *args, bq=hbq, bk=hbk,
                        q_out=s["yq"], k_out=s["yk"], **gopt)

    def gbwd(i):
        s = sets[i]
        qk.qknr_bwd_opt(s["q"], s["k"], hwq, hwk, s["pos"], s["dyq"], s["dyk"], *args,
                        bias_grads=True, dq=s["dq"], dk=s["dk"], dwq=hg[0], dwk=hg[1], dbq=hg[2],
                        dbk=hg[3], workspace=gws, **gopt)

    out["groups_head_weights"] = dict(timed_pair(gfwd, gbwd), norm_groups=[gq, hkv])

    # Layerwise QK-Norm (every q head one group, every k head another) with
    # [H, D] weights and biases: within one wave stage for the Qwen-shaped
    # heads (the wave kernel); across the stages of a token for the 7B-shaped
    # ones (the whole-token kernel).
    lopt = dict(flags=qk.QKNR_FLAG_HEAD_WEIGHTS, norm_groups=(hq, hkv))
    lws = torch.zeros(max(16, qk.qknr_bwd_opt_workspace_bytes(T, hq, hkv, D, w.rotary_dim, dt,
                                                              **lopt)), dtype=torch.uint8,
                      device=dev)

    def lwfwd(i):
        s = sets[i]
        qk.qknr_fwd_opt(s["q"], s["k"], hwq, hwk, s["pos"], *args, bq=hbq, bk=hbk,
                        q_out=s["yq"], k_out=s["yk"], **lopt)

    def lwbwd(i):
        s = sets[i]
        qk.qknr_bwd_opt(s["q"], s["k"], hwq, hwk, s["pos"], s["dyq"], s["dyk"], *args,
                        bias_grads=True, dq=s["dq"], dk=s["dk"], dwq=hg[0], dwk=hg[1], dbq=hg[2],
                        dbk=hg[3], workspace=lws, **lopt)

    out["layerwise_head_weights"] = dict(timed_pair(lwfwd, lwbwd), norm_groups=[hq, hkv])
    del lws

    # decode: B sequences, one new token each, K into a paged cache
    dec = {}
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    nslots = 256 * 1024
    cache = torch.zeros(nslots, hkv, D, dtype=dt, device=dev)
    for B in (1, 64, 256):
        q = torch.randn(B, hq, D, device=dev, generator=gen).to(dt)
        kk = torch.randn(B, hkv, D, device=dev, generator=gen).to(dt)
        pos = torch.randint(0, 262144, (B,), device=dev, generator=gen, dtype=torch.int32)
        slots = torch.randperm(nslots, device=dev, generator=gen)[:B].to(torch.int64)
        yq = torch.empty_like(q)

        def dstep():
            qk.qknr_fwd_ex(q, kk, base["wq"], base["wk"], pos, *args, q_out=yq, k_out=cache,
                           k_out_slots=slots)

        us = graph_time([dstep] * 32, max(4, k // 8), stream)
        byts = B * (2 * (hq + hkv) * D * q.element_size() + 4 + 8)
        dec["B%d" % B] = {"us": round(us, 3), "alg_bytes": byts,
                          "alg_GBps": round(byts / us / 1e3, 1)}
    out["decode_paged_k"] = dict(dec, cache_slots=nslots, positions="uniform in [0, 262144)")

    # decode with the group norms of the groups row above ([H, D] weights and
    # biases), K into the same paged cache: the norm-group kernels
    decg = {}
    for B in (1, 64, 256):
        q = torch.randn(B, hq, D, device=dev, generator=gen).to(dt)
        kk = torch.randn(B, hkv, D, device=dev, generator=gen).to(dt)
        pos = torch.randint(0, 262144, (B,), device=dev, generator=gen, dtype=torch.int32)
        slots = torch.randperm(nslots, device=dev, generator=gen)[:B].to(torch.int64)
        yq = torch.empty_like(q)

        def gstep():
            qk.qknr_fwd_opt(q, kk, hwq, hwk, pos, *args, bq=hbq, bk=hbk, q_out=yq, k_out=cache,
                            k_out_slots=slots, **gopt)

        us = graph_time([gstep] * 32, max(4, k // 8), stream)
        byts = B * (2 * (hq + hkv) * D * q.element_size() + 4 + 8)
        decg["B%d" % B] = {"us": round(us, 3), "alg_bytes": byts,
                           "alg_GBps": round(byts / us / 1e3, 1)}
    out["decode_groups_paged_k"] = dict(decg, norm_groups=[gq, hkv])

    # What bounds a decode step: the same graph replays of a kernel that does
    # nothing (a dispatch), and of a plain copy of the step's Q and K bytes
    # (one load round trip, then the stores; one workgroup up to 16 KiB)
    from qk_norm_rope_amd import bench_helpers as bh
    floor = {"empty_kernel_us": round(graph_time([lambda: bh.empty()] * 32, max(4, k // 8),
                                                 stream), 3)}
    for B in (1, 64, 256):
        src = torch.empty(B * (hq + hkv) * D, dtype=dt, device=dev)
        dst = torch.empty_like(src)
        us = graph_time([lambda src=src, dst=dst: bh.copy(src, dst)] * 32, max(4, k // 8), stream)
        floor["copy_B%d_us" % B] = round(us, 3)
    out["decode_floor"] = floor

    # Device Best-Fit-Decreasing packing (the data step that makes packed
    # position ids): the packed workload's document draw into 32768-token
    # buffers, and a larger mix; graph replays of back-to-back calls.
    from workloads import bfd as host_bfd, configs as wcfg, gen as wgen
    pw = wcfg.get("packed")
    docs = host_bfd.draw_lengths(wgen.rng(pw.seed, wgen.S_DOCS), pw.doc_len_min, pw.doc_len_max,
                                 pool_tokens=8 * pw.tokens)
    big = np.clip(np.rint(np.exp(np.random.default_rng(5).uniform(np.log(16), np.log(4096), 4000))),
                  16, 4096)
    packs = {}
    for name, lengths, cap, max_bins in (("packed_workload_docs", docs, pw.tokens, 64),
                                         ("4000_docs_into_4096", big, 4096, 2048)):
        lt = torch.from_numpy(np.asarray(lengths, np.int32)).to(dev)
        nd = int(lt.shape[0])
        pws = torch.empty(max(16, int(qk.lib.qknr_bfd_workspace_bytes(nd, max_bins))),
                          dtype=torch.uint8, device=dev)

        def pack(lt=lt, cap=cap, max_bins=max_bins, pws=pws):
            qk.qknr_bfd_pack(lt, cap, max_bins, workspace=pws)

        us = graph_time([pack] * 8, max(4, k // 16), stream)
        r = qk.qknr_bfd_pack(lt, cap, max_bins, workspace=pws)
        torch.cuda.synchronize()
        packs[name] = {"us": round(us, 2), "docs": nd, "capacity": cap,
                       "bins": int(r["counts"][0]), "status": int(r["status"][0])}
    out["bfd_pack"] = packs
    return out


def host_bits(t):
    """A device tensor's storage bits on the host (uint16 for bf16)."""
    import numpy as np
    import torch

    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class Bench:
    """Inputs, rotated sets and the timing protocol of one workload."""

    def __init__(self, qk, w, dev, stream):
        import numpy as np
        import torch

        from workloads import gen

        self.qk, self.w, self.stream = qk, w, stream
        inp = gen.make_inputs(w, backward=w.backward)

        def to_dev(key, v):
            if key == "pos":
                return torch.from_numpy(np.ascontiguousarray(v)).to(dev)
            if w.dtype == "bf16":
                return torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(np.ascontiguousarray(v)).to(dev)

        self.base = {key: to_dev(key, v) for key, v in inp.items()}
        del inp
        set_bytes = w.fwd_bytes() + (w.bwd_bytes() if w.backward else 0)
        self.nsets = max(3, min(16, -(-2 * MALL_BYTES // set_bytes) + 1))
        self.sets = []
        for i in range(self.nsets):
            s = {key: (t if i == 0 or key in ("wq", "wk", "pos") else t.clone())
                 for key, t in self.base.items()}
            outs = (("yq", "q"), ("yk", "k"))
            if w.backward:
                outs += (("dq", "q"), ("dk", "k"), ("dwq", "wq"), ("dwk", "wk"))
            for key, src in outs:
                s[key] = torch.empty_like(s[src])
            self.sets.append(s)
        self.ws = torch.zeros(max(16, qk.qknr_bwd_workspace_bytes(w.tokens, w.hq, w.hkv, w.head_dim,
                                                                  self.base["q"].dtype)),
                              dtype=torch.uint8, device=dev)
        self.args = (w.rotary_dim, w.eps, w.theta)

    def fwd(self, s):
        self.qk.qknr_fwd(s["q"], s["k"], s["wq"], s["wk"], s["pos"], *self.args, q_out=s["yq"],
                         k_out=s["yk"])

    def bwd(self, s):
        self.qk.qknr_bwd(s["q"], s["k"], s["wq"], s["wk"], s["pos"], s["dyq"], s["dyk"], *self.args,
                         dq=s["dq"], dk=s["dk"], dwq=s["dwq"], dwk=s["dwk"], workspace=self.ws)

    def step(self, i):
        """Step i: the forward of set i, then the backward of set i - 1."""
        n = self.nsets
        self.fwd(self.sets[i % n])
        if self.w.backward:
            self.bwd(self.sets[(i - 1) % n])

    def timed(self, fn, k):
        """fn(i) for i < k between two HIP events on the launch stream, with a
        synchronisation on each side; average microseconds per call."""
        import torch

        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(self.stream)
        for i in range(k):
            fn(i)
        t1.record(self.stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e3 / k

    def settle(self, settle_ms):
        """Untimed steps until at least settle_ms of GPU time has passed."""
        n, gpu_ms = 0, 0.0
        while gpu_ms < settle_ms and n < 100000:
            batch = 20
            gpu_ms += self.timed(lambda i: self.step(n + i), batch) * batch * 1e-3
            n += batch
        return {"gpu_ms": round(gpu_ms, 2), "steps": n}

    def run(self, steps, warmup, settle_ms=SETTLE_MS):
        w = self.w
        out = {"clock_settle": self.settle(settle_ms)}
        for i in range(warmup):
            self.step(i)
        step_us = self.timed(self.step, steps)
        fwd_us = self.timed(lambda i: self.fwd(self.sets[i % self.nsets]), steps)
        bwd_us = self.timed(lambda i: self.bwd(self.sets[i % self.nsets]), steps) if w.backward else 0.0
        out.update(step_us=step_us, fwd_us=fwd_us, bwd_us=bwd_us)
        return out

    def summary(self, r, steps, warmup):
        """The metric object of one workload from run()'s timings."""
        w = self.w
        kern = {"fwd_us": round(r["fwd_us"], 3), "fwd_alg_bytes": w.fwd_bytes(),
                "fwd_alg_GBps": round(w.fwd_bytes() / r["fwd_us"] / 1e3, 1)}
        if w.backward:
            kern.update(bwd_us=round(r["bwd_us"], 3), bwd_alg_bytes=w.bwd_bytes(),
                        bwd_alg_GBps=round(w.bwd_bytes() / r["bwd_us"] / 1e3, 1),
                        bwd_launches="qknr_kernel<bwd> + qknr_dw_finalize_kernel")
            dom_bytes, dom_us, dom_name = w.bwd_bytes(), r["bwd_us"], "qknr_bwd"
        else:
            dom_bytes, dom_us, dom_name = w.fwd_bytes(), r["fwd_us"], "qknr_fwd"
        achieved = dom_bytes / (dom_us * 1e-6) / 1e9
        traffic = traffic_from_counters(w.name) if w.backward else None
        calls = r["fwd_us"] + r["bwd_us"]
        return {
            "value": round(w.tokens / (r["step_us"] * 1e-6), 1),
            "unit": "tokens/s",
            "ms_per_step": round(r["step_us"] * 1e-3, 6),
            "steps": steps, "warmup": warmup,
            "clock_settle": r["clock_settle"],
            "step_over_calls": round(r["step_us"] / calls, 4),
            "config": {"workload": w.description, "name": w.name, "tokens": w.tokens, "hq": w.hq,
                       "hkv": w.hkv, "head_dim": w.head_dim, "rotary_dim": w.rotary_dim,
                       "io_dtype": w.dtype, "eps": w.eps, "theta": w.theta,
                       "passes": "fwd+bwd" if w.backward else "fwd", "rotated_sets": self.nsets},
            "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": round(achieved, 1),
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBPS, 4),
                         "traffic": None if traffic is None else round(traffic),
                         "alg_bytes": dom_bytes,
                         "traffic_source": ("profiles/counters.json: rocprofv3 --pmc FETCH_SIZE and "
                                            "WRITE_SIZE of the same command, copy-calibrated, "
                                            "kernel source %s" % kernel_hash())
                         if traffic is not None else "no committed counters for this kernel source",
                         "traffic_GBps": None if traffic is None else round(traffic / (dom_us * 1e3), 1)},
            "kernels": kern,
        }


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU component "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import qk_norm_rope_amd as qk
    from qk_norm_rope_amd import bench_helpers as bh
    from workloads import configs

    w = configs.get(a.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    main_b = Bench(qk, w, dev, stream)
    second = None if a.second == "none" or a.second == a.workload else configs.get(a.second)

    # the workloads back to back: settle, warmup, timed steps, per-call times
    r = main_b.run(a.steps, a.warmup, a.settle_ms)
    head = main_b.summary(r, a.steps, a.warmup)
    sets = main_b.sets
    # the GPU's outputs of set 0 for the parity statistics of the CPU leg
    main_b.fwd(sets[0])
    if w.backward:
        main_b.bwd(sets[0])
    torch.cuda.synchronize()
    gpu_out = {key: host_bits(sets[0][key])
               for key in (("yq", "yk", "dq", "dk", "dwq", "dwk") if w.backward else ("yq", "yk"))}

    # Each call alone, cold: a 1 GiB flush (four times the Infinity Cache)
    # before every call, outside the events that bracket the call; median,
    # p10 and p90 over the repetitions (the events add their own small gap).
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def cold(fn, reps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for i in range(reps):
            bh.flush(flush, i)
            ev[i][0].record(stream)
            fn(sets[i % len(sets)])
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        t = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)
        pick = lambda f: round(t[min(len(t) - 1, int(f * len(t)))], 3)  # noqa: E731
        return {"median_us": pick(0.5), "p10_us": pick(0.1), "p90_us": pick(0.9), "reps": reps}

    head["kernels"]["cold_fwd"] = cold(main_b.fwd, a.cold_reps)
    if w.backward:
        head["kernels"]["cold_bwd"] = cold(main_b.bwd, a.cold_reps)
    del flush

    # Plain streams as context: a copy moving the forward's bytes (read half,
    # write half), two reads and one write of the backward's bytes, and a copy
    # of 1 GiB.
    def stream_rate(nbuf, nbytes, fn, reps=30):
        nrot = max(3, -(-2 * MALL_BYTES // (nbuf * nbytes)) + 1)   # rotate past the Infinity Cache
        bufs = [[torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
                for _ in range(nrot)]
        for i, b in enumerate(bufs):
            for j, x in enumerate(b[:-1]):
                bh.flush(x, nbuf * i + j)
            fn(b)
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        c0.record(stream)
        for i in range(reps):
            fn(bufs[i % nrot])
        c1.record(stream)
        torch.cuda.synchronize()
        return nbuf * nbytes * reps / (c0.elapsed_time(c1) * 1e-3) / 1e9

    half = (w.fwd_bytes() // 2) // 16 * 16
    copy_fwd = stream_rate(2, half, lambda b: bh.copy(b[0], b[1]))
    stream2_bwd = None
    if w.backward:
        third = (w.bwd_bytes() // 3) // 16 * 16
        stream2_bwd = stream_rate(3, third, lambda b: bh.stream2(b[0], b[1], b[2]))
    copy_1g = stream_rate(2, 1 << 30, lambda b: bh.copy(b[0], b[1]), reps=10)

    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "clock_settle": head["clock_settle"],
        "ms_per_step": head["ms_per_step"],
        "step_over_calls": head["step_over_calls"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "storage_dtype": w.dtype,
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "kernels": head["kernels"],
        "copy_GBps": round(copy_1g, 1),
        "copy_GBps_at_fwd_bytes": round(copy_fwd, 1),
        "stream2_GBps_at_bwd_bytes": None if stream2_bwd is None else round(stream2_bwd, 1),
    }
    if w.backward and not a.no_variants:
        out["variants"] = measure_variants(qk, w, main_b.base, sets, a.steps, stream)
    del main_b, sets
    torch.cuda.empty_cache()
    if second is not None:
        sb = Bench(qk, second, dev, stream)
        out["second_workload"] = sb.summary(sb.run(a.steps, a.warmup, a.settle_ms), a.steps,
                                            a.warmup)
        del sb
        torch.cuda.empty_cache()
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, a.cpu_seconds, gpu_out)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

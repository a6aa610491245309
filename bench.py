#!/usr/bin/env python3
"""Benchmark of the fused QK-Norm + RoPE forward + backward on one MI355X.

A step is one forward and one backward (the whole hot path) over one batch of
the chosen workload; the default workload is the Qwen2.5-0.5B-shaped one
(8 x 4096 tokens, 14 Q / 2 KV heads, head_dim 64, bf16 storage, fp32
arithmetic).  Inputs are resident in HBM before timing starts.  Several
complete input/output sets are rotated so that the bytes touched between two
uses of a set exceed the 256 MB Infinity Cache: every step reads its inputs
from HBM.

Prints one JSON line: throughput (tokens/s over the timed steps), the roofline
of the dominant call (the backward: its main kernel plus the small dw
finalize kernel), timed over K back-to-back launches between HIP events on
the stream it runs on, and the oracle's throughput on the host cores as a CPU
baseline.  A "variants" object times the extended entry points on the same
shape (Q/K as views of a fused QKV buffer rewritten in place; interleaved
pairs), the dense calls the same way for reference, and decode steps that
write K through a slot map into a paged cache; those per-call times come from
HIP-graph replays, so the Python binding's host time does not hide short
kernels.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload qwen05|packed|7b|long|tiny]
                    [--no-cpu-baseline] [--no-variants]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QK-Norm+RoPE fwd+bwd tokens/s and achieved HBM GB/s (% of peak), 1 GPU"
HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, AMD public specification
MALL_BYTES = 256 << 20      # Infinity Cache
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
KERNEL_SRC = os.path.join(ROOT, "qk_norm_rope_amd", "csrc", "qknr.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed steps first; the GPU needs ~30 ms of work to reach steady clocks")
    ap.add_argument("--workload", default="qwen05")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--cold-reps", type=int, default=100,
                    help="repetitions of each call timed alone after a cache flush")
    return ap.parse_args()


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def traffic_from_counters(name: str, w):
    """HBM bytes of one backward call (main kernel + dw finalize) from the
    committed rocprofv3 --pmc readings (FETCH_SIZE and WRITE_SIZE in KiB per
    dispatch, each scaled by what the counter reads for a copy of known
    size), or None if there are none for the current kernel source."""
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


def cpu_baseline(w, budget_s: float):
    """The oracle, as it stands, on the host cores: forward + backward of the
    workload's first tokens, repeated until about `budget_s` CPU-seconds."""
    import numpy as np

    import oracle
    from workloads import gen

    try:
        cores = max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        cores = 4
    n_tok = min(w.tokens, 8192)
    inp = gen.make_inputs(w, 0, n_tok, backward=True)
    dec = lambda a: oracle.decode(a, w.dtype)  # noqa: E731
    q, k, wq, wk = dec(inp["q"]), dec(inp["k"]), dec(inp["wq"]), dec(inp["wk"])
    dyq, dyk = dec(inp["dyq"]), dec(inp["dyk"])
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.fwd(q, k, wq, wk, inp["pos"], w.rotary_dim, w.eps, w.theta, threads=cores)
        if w.backward:
            oracle.bwd(q, k, wq, wk, inp["pos"], dyq, dyk, w.rotary_dim, w.eps, w.theta,
                       threads=cores)
        reps += 1
        el = time.perf_counter() - t0
        if el * cores >= budget_s or reps >= 200:
            break
    # one thread, on the first 1024 tokens, for about a tenth of the budget
    n1 = min(n_tok, 1024)
    sl = lambda a: a[:n1]  # noqa: E731
    reps1 = 0
    t0 = time.perf_counter()
    while True:
        oracle.fwd(sl(q), sl(k), wq, wk, inp["pos"][:n1], w.rotary_dim, w.eps, w.theta, threads=1)
        if w.backward:
            oracle.bwd(sl(q), sl(k), wq, wk, inp["pos"][:n1], sl(dyq), sl(dyk), w.rotary_dim,
                       w.eps, w.theta, threads=1)
        reps1 += 1
        el1 = time.perf_counter() - t0
        if el1 >= budget_s / 10 or reps1 >= 200:
            break
    del np
    return {"value": reps * n_tok / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "%s: fwd%s of tokens [0, %d) x %d repetitions, fp64 C oracle, %d threads, "
                      "%.1f s wall" % (w.name, "+bwd" if w.backward else "", n_tok, reps, cores, el),
            "single_thread": {"value": reps1 * n1 / el1, "unit": "tokens/s",
                              "sample": "tokens [0, %d) x %d repetitions, 1 thread, %.1f s"
                                        % (n1, reps1, el1)}}


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
    into a paged cache [slots, hkv, D]; launch-latency bound; also with the
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


def main():
    a = parse()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU component "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import qk_norm_rope_amd as qk
    from qk_norm_rope_amd import bench_helpers as bh
    from workloads import configs, gen

    w = configs.get(a.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = gen.make_inputs(w, backward=True)

    def to_dev(key, v):
        if key == "pos":
            return torch.from_numpy(np.ascontiguousarray(v)).to(dev)
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(v)).to(dev)

    base = {key: to_dev(key, v) for key, v in inp.items()}
    set_bytes = w.fwd_bytes() + (w.bwd_bytes() if w.backward else 0)
    nsets = max(2, min(16, -(-2 * MALL_BYTES // set_bytes) + 1))
    sets = []
    for i in range(nsets):
        s = {key: (t if i == 0 or key in ("wq", "wk", "pos") else t.clone()) for key, t in base.items()}
        s["yq"] = torch.empty_like(s["q"])
        s["yk"] = torch.empty_like(s["k"])
        s["dq"] = torch.empty_like(s["q"])
        s["dk"] = torch.empty_like(s["k"])
        s["dwq"] = torch.empty_like(s["wq"])
        s["dwk"] = torch.empty_like(s["wk"])
        sets.append(s)
    ws = torch.zeros(max(16, qk.qknr_bwd_workspace_bytes(w.tokens, w.hq, w.hkv, w.head_dim,
                                                          base["q"].dtype)),
                     dtype=torch.uint8, device=dev)
    args = (w.rotary_dim, w.eps, w.theta)
    stream = torch.cuda.current_stream(dev)

    def fwd(s):
        qk.qknr_fwd(s["q"], s["k"], s["wq"], s["wk"], s["pos"], *args, q_out=s["yq"], k_out=s["yk"])

    def bwd(s):
        qk.qknr_bwd(s["q"], s["k"], s["wq"], s["wk"], s["pos"], s["dyq"], s["dyk"], *args,
                    dq=s["dq"], dk=s["dk"], dwq=s["dwq"], dwk=s["dwk"], workspace=ws)

    def step(s):
        fwd(s)
        if w.backward:
            bwd(s)

    def timed(fn, k):
        """Run fn on the rotated sets k times between two HIP events recorded
        on the launch stream; returns average microseconds per call."""
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(k):
            fn(sets[i % nsets])
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e3 / k

    for i in range(a.warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()

    # Timed region: exactly K steps (forward + backward), back to back, with
    # synchronisation and an event on each side.
    step_us = timed(step, a.steps)
    ms_per_step = step_us * 1e-3
    tokens_per_s = w.tokens / (ms_per_step * 1e-3)

    # Per-call durations for the roofline: K back-to-back launches of each
    # call between two events on the same stream (no events between
    # launches, which would add their own gaps).
    fwd_us = timed(fwd, a.steps)
    bwd_us = timed(bwd, a.steps) if w.backward else None
    fwd_gbps = w.fwd_bytes() / (fwd_us * 1e-6) / 1e9
    kern = {"fwd_us": round(fwd_us, 3), "fwd_alg_GBps": round(fwd_gbps, 1),
            "fwd_alg_bytes": w.fwd_bytes()}
    if w.backward:
        bwd_gbps = w.bwd_bytes() / (bwd_us * 1e-6) / 1e9
        kern.update({"bwd_us": round(bwd_us, 3), "bwd_alg_GBps": round(bwd_gbps, 1),
                     "bwd_alg_bytes": w.bwd_bytes(),
                     "bwd_launches": "qknr_kernel<bwd> + qknr_dw_finalize_kernel"})
        dom_bytes, dom_us, dom_name = w.bwd_bytes(), bwd_us, "qknr_bwd"
    else:
        dom_bytes, dom_us, dom_name = w.fwd_bytes(), fwd_us, "qknr_fwd"
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    traffic = traffic_from_counters(w.name, w) if w.backward else None

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
            fn(sets[i % nsets])
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        t = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)
        pick = lambda f: round(t[min(len(t) - 1, int(f * len(t)))], 3)  # noqa: E731
        return {"median_us": pick(0.5), "p10_us": pick(0.1), "p90_us": pick(0.9), "reps": reps}

    kern["cold_fwd"] = cold(fwd, a.cold_reps)
    if w.backward:
        kern["cold_bwd"] = cold(bwd, a.cold_reps)
    del flush

    # Achievable copy bandwidth as context: a copy moving the forward's bytes
    # (read half, write half), then 1 GiB read + 1 GiB write.
    half = (w.fwd_bytes() // 2) // 16 * 16
    ncp = max(3, -(-2 * MALL_BYTES // (2 * half)) + 1)   # rotate past the Infinity Cache
    csrc = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(ncp)]
    cdst = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(ncp)]
    for i in range(ncp):
        bh.flush(csrc[i], i)
        bh.copy(csrc[i], cdst[i])
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for i in range(30):
        bh.copy(csrc[i % ncp], cdst[i % ncp])
    c1.record(stream)
    torch.cuda.synchronize()
    copy_fwd_size_gbps = 2 * half * 30 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del csrc, cdst
    # The same for the backward's shape: two reads and one write of a third of
    # its bytes each.
    stream2_bwd_size_gbps = None
    if w.backward:
        third = (w.bwd_bytes() // 3) // 16 * 16
        nsr = max(3, -(-2 * MALL_BYTES // (3 * third)) + 1)
        sa = [torch.empty(third, dtype=torch.uint8, device=dev) for _ in range(nsr)]
        sb = [torch.empty(third, dtype=torch.uint8, device=dev) for _ in range(nsr)]
        sd = [torch.empty(third, dtype=torch.uint8, device=dev) for _ in range(nsr)]
        for i in range(nsr):
            bh.flush(sa[i], 2 * i)
            bh.flush(sb[i], 2 * i + 1)
            bh.stream2(sa[i], sb[i], sd[i])
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for i in range(30):
            bh.stream2(sa[i % nsr], sb[i % nsr], sd[i % nsr])
        c1.record(stream)
        torch.cuda.synchronize()
        stream2_bwd_size_gbps = 3 * third * 30 / (c0.elapsed_time(c1) * 1e-3) / 1e9
        del sa, sb, sd
    # Achievable copy bandwidth as context (1 GiB read + 1 GiB write).
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    bh.flush(src, 1)
    for _ in range(3):
        bh.copy(src, dst)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        bh.copy(src, dst)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * n * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.description, "name": w.name, "tokens": w.tokens, "hq": w.hq,
                   "hkv": w.hkv, "head_dim": w.head_dim, "rotary_dim": w.rotary_dim,
                   "io_dtype": w.dtype, "eps": w.eps, "theta": w.theta,
                   "passes": "fwd+bwd" if w.backward else "fwd", "rotated_sets": nsets},
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None if traffic is None else round(traffic), "alg_bytes": dom_bytes,
                     # counter bytes (FETCH_SIZE + WRITE_SIZE, copy-calibrated) over the same time
                     "traffic_GBps": None if traffic is None else round(traffic / (dom_us * 1e3), 1)},
        "kernels": kern,
        "copy_GBps": round(copy_gbps, 1),
        "copy_GBps_at_fwd_bytes": round(copy_fwd_size_gbps, 1),
        "stream2_GBps_at_bwd_bytes": (round(stream2_bwd_size_gbps, 1)
                                      if stream2_bwd_size_gbps is not None else None),
    }
    if w.backward and not a.no_variants:
        out["variants"] = measure_variants(qk, w, base, sets, a.steps, stream)
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

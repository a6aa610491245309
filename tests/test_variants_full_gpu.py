"""Full-size parity of the extended entry points, in the launch configurations
the benchmark times: the Qwen2.5-0.5B-shaped and 7B-shaped workloads (32768
tokens) with Q/K as views of a fused QKV buffer rewritten in place,
interleaved pairs, QK-LayerNorm with biases, a frequency table and an
attention factor, and norm groups (GQA-sized for q, layerwise for k) with
[H, D] weights and biases.  The GPU runs every row, and every output element
is compared with the oracle, chunk by chunk (y, dq, dk per 4096-token chunk;
the weight and bias gradients against the oracle summed over every row).
Same tolerance rules as the dense path (helpers.py); the count of elements
beyond a strict 2 ulp is printed per tensor.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from helpers import brief, compare, gpu_values, merge_stats, to_device
from workloads import configs, gen

pytestmark = pytest.mark.gpu

try:
    THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
except AttributeError:  # pragma: no cover
    THREADS = 4

IL, LN, HW = 1, 8, 16   # library flag bits
CHUNK = 4096


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def qk():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import qk_norm_rope_amd
    torch.cuda.set_device(0)
    return qk_norm_rope_amd


_INPUTS = {}


def inputs(name):
    if name not in _INPUTS:
        w = configs.get(name)
        say("generating", name)
        _INPUTS[name] = (w, gen.make_inputs(w, backward=True))
    return _INPUTS[name]


def oracle_args(inp, dtype, wq, wk):
    dec = lambda a: oracle.decode(a, dtype)  # noqa: E731
    return dec, dec(wq), dec(wk)


def check(w, inp, got, wq, wk, flags, what, bq=None, bk=None, table=None, attn=1.0,
          groups=None):
    """got: device tensors yq, yk, dq, dk, dwq, dwk[, dbq, dbk] of the full run.
    Every element of y, dq and dk is compared, a 4096-token chunk at a time,
    inside the loop that sums the oracle's weight (and bias) gradients over
    every row."""
    dt = w.dtype
    dec, owq, owk = oracle_args(inp, dt, wq, wk)
    obq = None if bq is None else dec(bq)
    obk = None if bk is None else dec(bk)
    of = oracle.flags_of(interleaved=bool(flags & IL), layernorm=bool(flags & LN),
                         head_weights=bool(flags & HW))
    kw = dict(threads=THREADS, flags=of, inv_freq=table, attention_factor=attn, norm_groups=groups)
    say("oracle over every row", what)
    stats = {}
    tot = None
    for a in range(0, w.tokens, CHUNK):
        b = min(w.tokens, a + CHUNK)
        q, k = dec(inp["q"][a:b]), dec(inp["k"][a:b])
        yq, yk = oracle.fwd(q, k, owq, owk, inp["pos"][a:b], w.rotary_dim, w.eps, w.theta,
                            bq=obq, bk=obk, **kw)
        r = oracle.bwd(q, k, owq, owk, inp["pos"][a:b], dec(inp["dyq"][a:b]),
                       dec(inp["dyk"][a:b]), w.rotary_dim, w.eps, w.theta,
                       bias_grads=bq is not None, **kw)
        for key, o in (("yq", yq), ("yk", yk), ("dq", r[0]), ("dk", r[1])):
            st = compare(gpu_values(got[key][a:b], dt), o, dt, "%s:%s[%d:%d]" % (what, key, a, b))
            stats[key] = merge_stats(stats.get(key), st)
        part = r[2:]
        tot = list(part) if tot is None else [t + p for t, p in zip(tot, part)]
    names = ("dwq", "dwk", "dbq", "dbk")[: len(tot)]
    for key, o in zip(names, tot):
        stats[key] = compare(gpu_values(got[key], dt), o, dt, what + ":" + key, row_sum=True)
    say(what, {key: brief(v) for key, v in stats.items()})


WORKLOADS = ["qwen05", "7b"]


@pytest.mark.parametrize("name", WORKLOADS)
def test_full_fused_qkv_in_place(qk, name):
    """Q/K as views of [T, (hq + 2 hkv) D] buffers: the forward rewrites the Q
    and K columns in place, the backward writes dq/dk over the gradient
    buffer's columns; the V columns are left alone."""
    w, inp = inputs(name)
    T, hq, hkv, D, dt = w.tokens, w.hq, w.hkv, w.head_dim, w.dtype
    width = (hq + 2 * hkv) * D
    g = np.random.default_rng(3)
    v = gen.encode(g.standard_normal((T, hkv * D)), dt)
    say("case fused", name)
    x = to_device(np.concatenate([inp["q"].reshape(T, -1), inp["k"].reshape(T, -1), v], 1), dt)
    gbuf = to_device(np.concatenate([inp["dyq"].reshape(T, -1), inp["dyk"].reshape(T, -1), v], 1),
                     dt)
    wq, wk = to_device(inp["wq"], dt), to_device(inp["wk"], dt)
    pos = torch.from_numpy(inp["pos"]).cuda()
    view = lambda b, o, h: b[:, o: o + h * D].unflatten(1, (h, D))  # noqa: E731
    q, k = view(x, 0, hq), view(x, hq * D, hkv)
    gq, gk = view(gbuf, 0, hq), view(gbuf, hq * D, hkv)
    # backward first (it reads q, k before the forward overwrites them)
    _, _, dwq, dwk = qk.qknr_bwd_ex(q, k, wq, wk, pos, gq, gk, w.rotary_dim, w.eps, w.theta,
                                    dq=gq, dk=gk)
    qk.qknr_fwd_ex(q, k, wq, wk, pos, w.rotary_dim, w.eps, w.theta, q_out=q, k_out=k)
    torch.cuda.synchronize()
    assert torch.equal(x[:, (hq + hkv) * D:], to_device(v, dt))
    assert torch.equal(gbuf[:, (hq + hkv) * D:], to_device(v, dt))
    got = {"yq": q, "yk": k, "dq": gq, "dk": gk, "dwq": dwq, "dwk": dwk}
    check(w, inp, got, inp["wq"], inp["wk"], 0, "fused " + name)


@pytest.mark.parametrize("name", WORKLOADS)
def test_full_interleaved(qk, name):
    w, inp = inputs(name)
    dt = w.dtype
    d = {key: to_device(val, dt) for key, val in inp.items() if key != "pos"}
    pos = torch.from_numpy(inp["pos"]).cuda()
    say("case interleaved", name)
    yq, yk = qk.qknr_fwd_ex(d["q"], d["k"], d["wq"], d["wk"], pos, w.rotary_dim, w.eps, w.theta,
                            flags=IL)
    dq, dk, dwq, dwk = qk.qknr_bwd_ex(d["q"], d["k"], d["wq"], d["wk"], pos, d["dyq"], d["dyk"],
                                      w.rotary_dim, w.eps, w.theta, flags=IL)
    torch.cuda.synchronize()
    got = {"yq": yq, "yk": yk, "dq": dq, "dk": dk, "dwq": dwq, "dwk": dwk}
    check(w, inp, got, inp["wq"], inp["wk"], IL, "interleaved " + name)


@pytest.mark.parametrize("name", WORKLOADS)
def test_full_layernorm_bias_table(qk, name):
    """QK-LayerNorm, [D] biases, a frequency table (the formula divided by 4)
    and an attention factor of 1.1; the backward also writes the bias
    gradients."""
    w, inp = inputs(name)
    dt, D = w.dtype, w.head_dim
    g = np.random.default_rng(4)
    bq, bk = gen.encode(0.2 * g.standard_normal(D), dt), gen.encode(0.2 * g.standard_normal(D), dt)
    h = w.rotary_dim // 2
    table = w.theta ** (-2.0 * np.arange(h) / w.rotary_dim) / 4.0
    d = {key: to_device(val, dt) for key, val in inp.items() if key != "pos"}
    pos = torch.from_numpy(inp["pos"]).cuda()
    say("case layernorm + bias + table", name)
    yq, yk = qk.qknr_fwd_opt(d["q"], d["k"], d["wq"], d["wk"], pos, w.rotary_dim, w.eps,
                             w.theta, flags=LN, bq=to_device(bq, dt), bk=to_device(bk, dt),
                             inv_freq=table, attention_factor=1.1)
    dq, dk, dwq, dwk, dbq, dbk = qk.qknr_bwd_opt(d["q"], d["k"], d["wq"], d["wk"], pos, d["dyq"],
                                                 d["dyk"], w.rotary_dim, w.eps, w.theta,
                                                 flags=LN, bias_grads=True, inv_freq=table,
                                                 attention_factor=1.1)
    torch.cuda.synchronize()
    got = {"yq": yq, "yk": yk, "dq": dq, "dk": dk, "dwq": dwq, "dwk": dwk, "dbq": dbq, "dbk": dbk}
    check(w, inp, got, inp["wq"], inp["wk"], LN, "layernorm " + name, bq=bq, bk=bk, table=table,
          attn=1.1)


@pytest.mark.parametrize("name", WORKLOADS)
def test_full_groups_head_weights(qk, name):
    """Norm groups of hq / hkv q heads and of all hkv k heads, [H, D] weights
    and biases (the wave-level norm-group kernel: every group lies within one
    wave stage in both shapes); the backward writes [H, D] weight and bias
    gradients."""
    w, inp = inputs(name)
    dt, hq, hkv, D = w.dtype, w.hq, w.hkv, w.head_dim
    groups = (hq // hkv, hkv)
    g = np.random.default_rng(5)
    wq = gen.encode(1 + 0.1 * g.standard_normal((hq, D)), dt)
    wk = gen.encode(1 + 0.1 * g.standard_normal((hkv, D)), dt)
    bq = gen.encode(0.2 * g.standard_normal((hq, D)), dt)
    bk = gen.encode(0.2 * g.standard_normal((hkv, D)), dt)
    d = {key: to_device(inp[key], dt) for key in ("q", "k", "dyq", "dyk")}
    pos = torch.from_numpy(inp["pos"]).cuda()
    say("case groups + [H, D] weights", name, groups)
    yq, yk = qk.qknr_fwd_opt(d["q"], d["k"], to_device(wq, dt), to_device(wk, dt), pos,
                             w.rotary_dim, w.eps, w.theta, flags=HW, bq=to_device(bq, dt),
                             bk=to_device(bk, dt), norm_groups=groups)
    dq, dk, dwq, dwk, dbq, dbk = qk.qknr_bwd_opt(d["q"], d["k"], to_device(wq, dt),
                                                 to_device(wk, dt), pos, d["dyq"], d["dyk"],
                                                 w.rotary_dim, w.eps, w.theta, flags=HW,
                                                 bias_grads=True, norm_groups=groups)
    torch.cuda.synchronize()
    got = {"yq": yq, "yk": yk, "dq": dq, "dk": dk, "dwq": dwq, "dwk": dwk, "dbq": dbq, "dbk": dbk}
    check(w, inp, got, wq, wk, HW, "groups " + name, bq=bq, bk=bk, groups=groups)

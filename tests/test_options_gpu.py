"""Parity of qknr_fwd_opt / qknr_bwd_opt with the fp64 oracle: QK-LayerNorm,
[D] biases added after the weight (and their gradients), a caller frequency
table with an attention factor on cos and sin, each alone and combined with
the earlier options (interleaved pairs, parameter-free norm, strided views).
Same tolerance rules as the dense path (helpers.py).  The default options give
results bit-identical to the plain entry points.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from helpers import compare, gpu_values, to_device
from workloads import gen

pytestmark = pytest.mark.gpu

try:
    THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
except AttributeError:  # pragma: no cover
    THREADS = 4

IL, FH, NW, LN = 1, 2, 4, 8   # QKNR_FLAG_INTERLEAVED, _FREQ_HEAD_DIM, _NO_WEIGHT, _LAYERNORM


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def qk():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import qk_norm_rope_amd
    torch.cuda.set_device(0)
    return qk_norm_rope_amd


def scaled_table(R, theta, factor, low=1.0, high=32.0, max_len=4096):
    """A frequency table of the "extension" kind: each frequency of the
    theta^(-2i/R) formula divided by a per-pair factor ramping from 1 (short
    wavelengths) to `factor` (long wavelengths), as position-interpolation
    schemes do.  Any finite table is valid input; this one is just realistic."""
    h = R // 2
    base = theta ** (-2.0 * np.arange(h) / R)
    wavelen = 2 * np.pi / base
    ramp = np.clip((max_len / wavelen - low) / (high - low), 0.0, 1.0)
    return base / (ramp * 1.0 + (1.0 - ramp) * factor)


def biases(seed, D, dtype):
    g = np.random.default_rng(seed)
    return gen.encode(0.2 * g.standard_normal(D), dtype), gen.encode(0.2 * g.standard_normal(D), dtype)


def oracle_ref(inp, dtype, R, eps, theta, flags, backward, bias=None, table=None, attn=1.0,
               bias_grads=False):
    dec = lambda a: oracle.decode(a, dtype)  # noqa: E731
    q, k = dec(inp["q"]), dec(inp["k"])
    D = q.shape[2]
    wq, wk = (np.ones(D), np.ones(D)) if flags & NW else (dec(inp["wq"]), dec(inp["wk"]))
    of = oracle.flags_of(interleaved=bool(flags & IL), freq_head_dim=bool(flags & FH),
                         layernorm=bool(flags & LN))
    bq, bk = (None, None) if bias is None else (dec(bias[0]), dec(bias[1]))
    yq, yk = oracle.fwd(q, k, wq, wk, inp["pos"], R, eps, theta, threads=THREADS, flags=of,
                        bq=bq, bk=bk, inv_freq=table, attention_factor=attn)
    out = {"yq": yq, "yk": yk}
    if backward:
        r = oracle.bwd(q, k, wq, wk, inp["pos"], dec(inp["dyq"]), dec(inp["dyk"]), R, eps, theta,
                       threads=THREADS, flags=of, inv_freq=table, attention_factor=attn,
                       bias_grads=bias_grads)
        out.update(zip(("dq", "dk", "dwq", "dwk", "dbq", "dbk"), r))
    return out


SHAPES = [  # dtype, D, R, T, hq, hkv
    ("bf16", 64, 64, 257, 14, 2),
    ("bf16", 128, 32, 131, 8, 2),
    ("bf16", 256, 128, 41, 3, 1),
    ("f32", 64, 48, 150, 5, 3),
    ("f32", 128, 128, 77, 4, 4),
    ("f32", 256, 16, 29, 2, 1),
    ("bf16", 128, 0, 1, 2, 6),   # no rotation, one token, more k heads than q heads
]

VARIANTS = {  # name: (flags, with biases, with a table, attention factor)
    "layernorm": (LN, False, False, 1.0),
    "bias": (0, True, False, 1.0),
    "table_attn": (0, False, True, 1.2),
    "layernorm_bias_table": (LN, True, True, 0.9),
    "ln_bias_interleaved_noweight": (LN | IL | NW, True, False, 1.0),
    "attn_only": (0, False, False, 1.5),
}


@pytest.mark.parametrize("variant", sorted(VARIANTS))
@pytest.mark.parametrize("dtype,D,R,T,hq,hkv", SHAPES)
def test_options_forward_backward(qk, variant, dtype, D, R, T, hq, hkv):
    flags, with_bias, with_table, attn = VARIANTS[variant]
    theta = 5e5
    what = "%s %s D=%d R=%d T=%d hq=%d hkv=%d" % (variant, dtype, D, R, T, hq, hkv)
    inp = gen.random_case(seed=D + R + T + flags, tokens=T, hq=hq, hkv=hkv, head_dim=D,
                          dtype=dtype, scale=1.3, max_pos=200000, backward=True)
    if flags & LN:
        # a per-row offset, so that the centring matters
        g = np.random.default_rng(T)
        for key, H in (("q", hq), ("k", hkv)):
            x = oracle.decode(inp[key], dtype) + 0.7 * g.standard_normal((T, H, 1))
            inp[key] = gen.encode(x, dtype)
    bias = biases(D + T, D, dtype) if with_bias else None
    table = scaled_table(R, theta, 8.0) if with_table else None
    say("case", what)
    d = {key: to_device(val, dtype) for key, val in inp.items() if key != "pos"}
    pos = torch.from_numpy(inp["pos"]).cuda()
    wq, wk = (None, None) if flags & NW else (d["wq"], d["wk"])
    bq, bk = (None, None) if bias is None else (to_device(bias[0], dtype), to_device(bias[1], dtype))
    yq, yk = qk.qknr_fwd_opt(d["q"], d["k"], wq, wk, pos, R, 1e-5, theta, flags=flags, bq=bq, bk=bk,
                             inv_freq=table, attention_factor=attn)
    dq, dk, dwq, dwk, dbq, dbk = qk.qknr_bwd_opt(
        d["q"], d["k"], wq, wk, pos, d["dyq"], d["dyk"], R, 1e-5, theta, flags=flags,
        bias_grads=with_bias, inv_freq=table, attention_factor=attn)
    torch.cuda.synchronize()
    o = oracle_ref(inp, dtype, R, 1e-5, theta, flags, True, bias=bias, table=table, attn=attn,
                   bias_grads=with_bias)
    for key, t in (("yq", yq), ("yk", yk), ("dq", dq), ("dk", dk)):
        compare(gpu_values(t, dtype), o[key], dtype, what + ":" + key)
    grads = [("dwq", dwq), ("dwk", dwk)] if not flags & NW else []
    grads += [("dbq", dbq), ("dbk", dbk)] if with_bias else []
    for key, t in grads:
        compare(gpu_values(t, dtype), o[key], dtype, what + ":" + key, row_sum=True)
    if flags & NW:
        assert dwq is None and dwk is None
    if not with_bias:
        assert dbq is None and dbk is None


def test_options_change_the_result(qk):
    """Each option moves the output away from the plain result by far more
    than the tolerance (so a kernel ignoring it would fail the parity test)."""
    dtype, D, R, T, hq, hkv, theta = "bf16", 128, 64, 64, 4, 2, 1e4
    inp = gen.random_case(seed=3, tokens=T, hq=hq, hkv=hkv, head_dim=D, dtype=dtype,
                          max_pos=5000, backward=False)
    say("case options change results")
    base = oracle_ref(inp, dtype, R, 1e-5, theta, 0, False)["yq"]
    bias = biases(1, D, dtype)
    for kw in (dict(flags=LN), dict(bias=bias), dict(table=scaled_table(R, theta, 4.0)),
               dict(attn=1.1)):
        flags = kw.pop("flags", 0)
        o = oracle_ref(inp, dtype, R, 1e-5, theta, flags, False, **kw)["yq"]
        assert np.abs(o - base).max() > 0.05, kw


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_default_options_equal_plain_entry_points(qk, dtype):
    """Default options (no flags, biases or table, factor 1) run the plain
    kernels: results are bit-identical to qknr_fwd / qknr_bwd."""
    T, hq, hkv, D, R = 199, 6, 2, 64, 64
    inp = gen.random_case(seed=21, tokens=T, hq=hq, hkv=hkv, head_dim=D, dtype=dtype,
                          max_pos=20000, backward=True)
    say("case opt == plain", dtype)
    d = {key: to_device(val, dtype) for key, val in inp.items() if key != "pos"}
    pos = torch.from_numpy(inp["pos"]).cuda()
    a = qk.qknr_fwd(d["q"], d["k"], d["wq"], d["wk"], pos, R, 1e-6, 1e4)
    b = qk.qknr_fwd_opt(d["q"], d["k"], d["wq"], d["wk"], pos, R, 1e-6, 1e4)
    ga = qk.qknr_bwd(d["q"], d["k"], d["wq"], d["wk"], pos, d["dyq"], d["dyk"], R, 1e-6, 1e4)
    gb = qk.qknr_bwd_opt(d["q"], d["k"], d["wq"], d["wk"], pos, d["dyq"], d["dyk"], R, 1e-6, 1e4)
    # a table equal to the formula and a factor of 1 change nothing either
    tab = 1e4 ** (-2.0 * np.arange(R // 2) / R)
    c = qk.qknr_fwd_opt(d["q"], d["k"], d["wq"], d["wk"], pos, R, 1e-6, 1e4, inv_freq=tab,
                        attention_factor=1.0)
    torch.cuda.synchronize()
    for x, y in zip(list(a) + list(ga), list(b) + list(gb[:4])):
        assert torch.equal(x, y)
    assert gb[4] is None and gb[5] is None
    for x, y in zip(a, c):
        assert torch.equal(x, y)


def test_options_on_fused_views_in_place(qk):
    """LayerNorm + biases + table on Q/K views of a fused QKV buffer, rotated
    in place; V untouched."""
    dtype, T, hq, hkv, D, R, theta = "bf16", 173, 8, 2, 128, 128, 1e6
    inp = gen.random_case(seed=8, tokens=T, hq=hq, hkv=hkv, head_dim=D, dtype=dtype,
                          max_pos=100000, backward=False)
    v = gen.encode(np.random.default_rng(2).standard_normal((T, hkv, D)), dtype)
    host = np.concatenate([inp["q"].reshape(T, -1), inp["k"].reshape(T, -1), v.reshape(T, -1)], 1)
    say("case options on fused views")
    buf = to_device(host, dtype)
    q = buf[:, : hq * D].unflatten(1, (hq, D))
    k = buf[:, hq * D: (hq + hkv) * D].unflatten(1, (hkv, D))
    bias = biases(5, D, dtype)
    table = scaled_table(R, theta, 16.0)
    qk.qknr_fwd_opt(q, k, to_device(inp["wq"], dtype), to_device(inp["wk"], dtype),
                    torch.from_numpy(inp["pos"]).cuda(), R, 1e-6, theta, flags=LN,
                    bq=to_device(bias[0], dtype), bk=to_device(bias[1], dtype), inv_freq=table,
                    attention_factor=1.05, q_out=q, k_out=k)
    torch.cuda.synchronize()
    o = oracle_ref(inp, dtype, R, 1e-6, theta, LN, False, bias=bias, table=table, attn=1.05)
    compare(gpu_values(q, dtype), o["yq"], dtype, "fused opt yq")
    compare(gpu_values(k, dtype), o["yk"], dtype, "fused opt yk")
    after = buf[:, (hq + hkv) * D:].cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(after, v.reshape(T, -1))


def test_binding_rejects_bad_options(qk):
    T, hq, hkv, D = 8, 2, 1, 64
    q = torch.zeros(T, hq, D, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(T, hkv, D, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(D, dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros(T, dtype=torch.int32, device="cuda")
    say("case option errors")
    with pytest.raises(ValueError):   # one bias only
        qk.qknr_fwd_opt(q, k, w, w, pos, 64, 1e-6, 1e4, bq=w)
    with pytest.raises(ValueError):   # table of the wrong length
        qk.qknr_fwd_opt(q, k, w, w, pos, 64, 1e-6, 1e4, inv_freq=[1.0] * 5)
    with pytest.raises(qk.QknrError):   # non-finite frequency
        qk.qknr_fwd_opt(q, k, w, w, pos, 64, 1e-6, 1e4, inv_freq=[float("nan")] * 32)
    with pytest.raises(qk.QknrError):   # non-finite factor
        qk.qknr_fwd_opt(q, k, w, w, pos, 64, 1e-6, 1e4, attention_factor=float("inf"))

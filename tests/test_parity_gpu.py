"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Every case draws seeded inputs, runs the library on the GPU and the oracle on
the host on the same stored values, and compares element by element under the
rules in helpers.py (fp32: 2e-5 absolute; bf16: 2 ulp of the oracle's rounded
value with a 2^-16 * row-RMS floor).
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


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def qk():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import qk_norm_rope_amd
    torch.cuda.set_device(0)
    return qk_norm_rope_amd


def dev_inputs(inp, dtype):
    d = {}
    for key, v in inp.items():
        d[key] = torch.from_numpy(np.ascontiguousarray(v)).cuda() if key == "pos" else to_device(v, dtype)
    return d


def run_gpu(qk, inp, dtype, R, eps, theta, backward):
    d = dev_inputs(inp, dtype)
    yq, yk = qk.qknr_fwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], R, eps, theta)
    out = {"yq": yq, "yk": yk}
    if backward:
        dq, dk, dwq, dwk = qk.qknr_bwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], d["dyq"],
                                       d["dyk"], R, eps, theta)
        out.update(dq=dq, dk=dk, dwq=dwq, dwk=dwk)
    torch.cuda.synchronize()
    return out


def run_oracle(inp, dtype, R, eps, theta, backward):
    dec = lambda a: oracle.decode(a, dtype)  # noqa: E731
    q, k, wq, wk = dec(inp["q"]), dec(inp["k"]), dec(inp["wq"]), dec(inp["wk"])
    yq, yk = oracle.fwd(q, k, wq, wk, inp["pos"], R, eps, theta, threads=THREADS)
    out = {"yq": yq, "yk": yk}
    if backward:
        dq, dk, dwq, dwk = oracle.bwd(q, k, wq, wk, inp["pos"], dec(inp["dyq"]), dec(inp["dyk"]),
                                      R, eps, theta, threads=THREADS)
        out.update(dq=dq, dk=dk, dwq=dwq, dwk=dwk)
    return out


def check_case(qk, inp, dtype, R, eps, theta, backward, what, plain_dw=False):
    """plain_dw: hold the fp32 weight gradients to the plain absolute bound
    instead of the one scaled by the vector's RMS."""
    say("case", what)
    g = run_gpu(qk, inp, dtype, R, eps, theta, backward)
    o = run_oracle(inp, dtype, R, eps, theta, backward)
    stats = {}
    for key in o:
        stats[key] = compare(gpu_values(g[key], dtype), o[key], dtype, "%s:%s" % (what, key),
                             row_sum=key.startswith("dw") and not plain_dw)
    if backward:
        for key in ("dq", "dk", "dwq", "dwk"):  # gradients are really there (non-zero)
            assert np.abs(o[key]).max() > 1e-3 and np.abs(gpu_values(g[key], dtype)).max() > 1e-3
    return stats


def test_tiny_config(qk):
    """The tiny fp32 configuration: every output, the weight gradients
    included, within the plain 2e-5 absolute bound."""
    w = configs.TINY
    inp = gen.make_inputs(w)
    st = check_case(qk, inp, w.dtype, w.rotary_dim, w.eps, w.theta, True, "tiny", plain_dw=True)
    say({k: brief(v) for k, v in st.items()})


@pytest.mark.parametrize("name", list(configs.ALL))
def test_config_slices(qk, name):
    """Each configuration's shapes, dtype and constants on 307 tokens (19 tiles
    of 16 and a ragged tail), taken from the middle of its token range so the
    positions are the configuration's own; forward and backward."""
    w = configs.get(name)
    n = min(307, w.tokens)
    t0 = min(w.tokens - n, 4000)
    inp = gen.make_inputs(w, t0, t0 + n, backward=True)
    check_case(qk, inp, w.dtype, w.rotary_dim, w.eps, w.theta, True, "%s[%d:%d]" % (name, t0, t0 + n))


# rotary widths: none, powers of two, and one whose half is not a power of two
# (48, 80, 240: 24, 40 and 120 frequencies per token)
SWEEP = []
for _dt in ("f32", "bf16"):
    for _D in (64, 128, 256):
        for _R in sorted({0, 16, 32, _D // 2, _D, {64: 48, 128: 80, 256: 240}[_D]}):
            if _R <= _D:
                SWEEP.append((_dt, _D, _R))


@pytest.mark.parametrize("dtype,D,R", SWEEP)
@pytest.mark.parametrize("T,hq,hkv", [(1, 1, 1), (37, 3, 1), (70, 5, 3)])
def test_sweep(qk, dtype, D, R, T, hq, hkv):
    inp = gen.random_case(seed=D + R + T, tokens=T, hq=hq, hkv=hkv, head_dim=D, dtype=dtype,
                          scale=1.5, max_pos=200000)
    check_case(qk, inp, dtype, R, 1e-5, 1e4 if R <= 32 else 5e5, True,
               "sweep %s D=%d R=%d T=%d hq=%d hkv=%d" % (dtype, D, R, T, hq, hkv))


@pytest.mark.parametrize("dtype,D,R,T,hq,hkv", [("bf16", 64, 64, 5, 1024, 1024),
                                                 ("f32", 256, 128, 3, 1024, 1024),
                                                 ("bf16", 128, 64, 9, 1024, 1),
                                                 ("bf16", 128, 128, 4, 1, 1024)])
def test_maximum_head_counts(qk, dtype, D, R, T, hq, hkv):
    """At the largest head counts the library takes (1024 per tensor, 2048
    rows per token): the token-block mapping's row -> token division holds."""
    inp = gen.random_case(seed=hq + hkv + D, tokens=T, hq=hq, hkv=hkv, head_dim=D, dtype=dtype,
                          scale=1.0, max_pos=100000)
    check_case(qk, inp, dtype, R, 1e-6, 1e4, True,
               "max heads %s D=%d R=%d T=%d hq=%d hkv=%d" % (dtype, D, R, T, hq, hkv))


@pytest.mark.parametrize("name", ["qwen05", "packed"])
def test_full_config_every_element(qk, name):
    """Full-size configuration, every output element and dw compared."""
    w = configs.get(name)
    inp = gen.make_inputs(w)
    st = check_case(qk, inp, w.dtype, w.rotary_dim, w.eps, w.theta, True, name)
    say({k: {kk: v[kk] for kk in ("max_ulp", "beyond_strict_2ulp")} for k, v in st.items()})


def _compare_chunks(w, gpu, keys, backward, what, chunk=4096):
    """Every element of the full-size outputs against the oracle, a chunk of
    tokens at a time (inputs regenerated per chunk); returns per-tensor
    statistics and, with the backward, the oracle's dw summed over every row."""
    dec = lambda a: oracle.decode(a, w.dtype)  # noqa: E731
    wq, wk = gen.weights(w)
    owq, owk = dec(wq), dec(wk)
    stats, dw = {}, None
    for a in range(0, w.tokens, chunk):
        b = min(w.tokens, a + chunk)
        inp = gen.make_inputs(w, a, b, backward=backward)
        q, k = dec(inp["q"]), dec(inp["k"])
        o = dict(zip(("yq", "yk"), oracle.fwd(q, k, owq, owk, inp["pos"], w.rotary_dim, w.eps,
                                               w.theta, threads=THREADS)))
        if backward:
            r = oracle.bwd(q, k, owq, owk, inp["pos"], dec(inp["dyq"]), dec(inp["dyk"]),
                           w.rotary_dim, w.eps, w.theta, threads=THREADS)
            o.update(dq=r[0], dk=r[1])
            dw = [r[2], r[3]] if dw is None else [dw[0] + r[2], dw[1] + r[3]]
        for key in keys:
            st = compare(gpu_values(gpu[key][a:b], w.dtype), o[key], w.dtype,
                         "%s:%s[%d:%d]" % (what, key, a, b))
            stats[key] = merge_stats(stats.get(key), st)
    return stats, dw


def test_full_config_7b_every_element(qk):
    """7B-shaped configuration at full size (4 x 8192 tokens, 32 + 8 heads of
    128, 1% outlier channels): every element of yq, yk, dq and dk compared
    with the oracle, and dw against the oracle summed over every row."""
    w = configs.LLAMA7B
    say("generating", w.name)
    inp = gen.make_inputs(w)
    d = dev_inputs(inp, w.dtype)
    del inp
    say("gpu", w.name)
    yq, yk = qk.qknr_fwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], w.rotary_dim, w.eps, w.theta)
    dq, dk, dwq, dwk = qk.qknr_bwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], d["dyq"], d["dyk"],
                                   w.rotary_dim, w.eps, w.theta)
    torch.cuda.synchronize()
    say("oracle over every row", w.name)
    stats, dw = _compare_chunks(w, dict(yq=yq, yk=yk, dq=dq, dk=dk), ("yq", "yk", "dq", "dk"),
                                True, "7b")
    stats["dwq"] = compare(gpu_values(dwq, w.dtype), dw[0], w.dtype, "7b:dwq", row_sum=True)
    stats["dwk"] = compare(gpu_values(dwk, w.dtype), dw[1], w.dtype, "7b:dwk", row_sum=True)
    say("7b", {k: brief(v) for k, v in stats.items()})


def test_full_config_long_forward_every_element(qk):
    """Long-context partial-RoPE forward at full size (131072 tokens, 64 + 8
    heads of 128, rotary_dim 32, positions up to 131071): every element of yq
    and yk compared with the oracle."""
    w = configs.LONG
    say("generating", w.name)
    inp = gen.make_inputs(w, backward=False)
    d = dev_inputs(inp, w.dtype)
    del inp
    say("gpu", w.name)
    yq, yk = qk.qknr_fwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], w.rotary_dim, w.eps, w.theta)
    torch.cuda.synchronize()
    del d
    say("oracle over every row", w.name)
    stats, _ = _compare_chunks(w, dict(yq=yq, yk=yk), ("yq", "yk"), False, "long")
    say("long", {k: brief(v) for k, v in stats.items()})


def test_many_rounds_of_two_block_waves_every_element(qk):
    """Qwen-shaped heads at more than four times the tokens (one sequence of
    33 x 4096 + 1 tokens), so that a persistent forward wave's share would pass
    16 stages and the forward launches waves of two two-stage token blocks in
    several workgroup rounds, the last wave holding only the final block, of a
    single token: every element of yq and yk (and of the backward's dq and dk,
    with dw over every row) against the oracle."""
    from dataclasses import replace as _replace
    w = _replace(configs.QWEN05, name="qwen05_many", batch=1, seq=33 * 4096 + 1)
    say("generating", w.name, w.tokens)
    inp = gen.make_inputs(w)
    d = dev_inputs(inp, w.dtype)
    del inp
    yq, yk = qk.qknr_fwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], w.rotary_dim, w.eps, w.theta)
    dq, dk, dwq, dwk = qk.qknr_bwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], d["dyq"], d["dyk"],
                                   w.rotary_dim, w.eps, w.theta)
    torch.cuda.synchronize()
    del d
    say("oracle over every row", w.name)
    stats, dw = _compare_chunks(w, dict(yq=yq, yk=yk, dq=dq, dk=dk), ("yq", "yk", "dq", "dk"),
                                True, w.name, chunk=16384)
    stats["dwq"] = compare(gpu_values(dwq, w.dtype), dw[0], w.dtype, "many:dwq", row_sum=True)
    stats["dwk"] = compare(gpu_values(dwk, w.dtype), dw[1], w.dtype, "many:dwk", row_sum=True)
    say(w.name, {k: brief(v) for k, v in stats.items()})


def _bits(t):
    """bf16 device tensor -> its uint16 bit patterns on the host."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def test_offsets_beyond_2_31_elements(qk):
    """A Q tensor of more than 2^31 elements (131109 tokens x 128 heads x 128,
    4.3 GB of bf16; K has 8 heads): byte offsets pass 2^31 at token 65536 and
    element offsets at token 131072.  Forward and backward run over every token;
    yq, yk, dq and dk are compared with the oracle on every element of the
    first tokens, of the tokens around both crossings and of the ragged end,
    and dw against the oracle summed over every row (4096-token chunks)."""
    T, hq, hkv, D, R, eps, theta = 131109, 128, 8, 128, 64, 1e-6, 1e4
    assert T * hq * D > 2 ** 31
    bf = torch.bfloat16
    g = torch.Generator(device="cuda")
    g.manual_seed(2031)
    say("case offsets beyond 2^31 elements: generating")
    q = torch.empty(T, hq, D, dtype=bf, device="cuda")
    dyq = torch.empty_like(q)
    for a in range(0, T, 16384):  # in slices, to bound the fp32 temporaries
        b = min(T, a + 16384)
        q[a:b] = (2 * torch.randn(b - a, hq, D, device="cuda", generator=g)).to(bf)
        dyq[a:b] = torch.randn(b - a, hq, D, device="cuda", generator=g).to(bf)
    k = (2 * torch.randn(T, hkv, D, device="cuda", generator=g)).to(bf)
    dyk = torch.randn(T, hkv, D, device="cuda", generator=g).to(bf)
    wq = (1 + 0.1 * torch.randn(D, device="cuda", generator=g)).to(bf)
    wk = (1 + 0.1 * torch.randn(D, device="cuda", generator=g)).to(bf)
    pos = (torch.arange(T, device="cuda") % 8192).to(torch.int32)
    say("gpu")
    yq, yk = qk.qknr_fwd(q, k, wq, wk, pos, R, eps, theta)
    dq, dk, dwq, dwk = qk.qknr_bwd(q, k, wq, wk, pos, dyq, dyk, R, eps, theta)
    torch.cuda.synchronize()
    dec = lambda a: oracle.decode(a, "bf16")  # noqa: E731
    owq, owk = dec(_bits(wq)), dec(_bits(wk))
    host_pos = pos.cpu().numpy()
    samples = [(0, 1024), (65536 - 512, 65536 + 512), (131072 - 512, T)]
    stats = {}
    dw = None
    say("oracle over every row")
    for a in range(0, T, 4096):
        b = min(T, a + 4096)
        sl = slice(a, b)
        oq, ok, ogq, ogk = (dec(_bits(t[sl])) for t in (q, k, dyq, dyk))
        r = oracle.bwd(oq, ok, owq, owk, host_pos[sl], ogq, ogk, R, eps, theta, threads=THREADS)
        dw = [r[2], r[3]] if dw is None else [dw[0] + r[2], dw[1] + r[3]]
        for s0, s1 in samples:
            lo, hi = max(a, s0), min(b, s1)
            if lo >= hi:
                continue
            part = slice(lo - a, hi - a)
            y = oracle.fwd(oq[part], ok[part], owq, owk, host_pos[lo:hi], R, eps, theta,
                           threads=THREADS)
            for key, got, want in (("yq", yq, y[0]), ("yk", yk, y[1]), ("dq", dq, r[0][part]),
                                   ("dk", dk, r[1][part])):
                st = compare(dec(_bits(got[lo:hi])), want, "bf16", "2^31:%s[%d:%d]" % (key, lo, hi))
                stats[key] = merge_stats(stats.get(key), st)
    stats["dwq"] = compare(dec(_bits(dwq)), dw[0], "bf16", "2^31:dwq", row_sum=True)
    stats["dwk"] = compare(dec(_bits(dwk)), dw[1], "bf16", "2^31:dwk", row_sum=True)
    say("2^31", {key: brief(v) for key, v in stats.items()})


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_extreme_positions(qk, dtype):
    """Largest and negative int32 positions (fp64 angles up to 2^31 rad)."""
    inp = gen.random_case(seed=99, tokens=12, hq=3, hkv=2, head_dim=128, dtype=dtype)
    inp["pos"] = np.array([0, 1, -1, -5, 2 ** 31 - 1, -2 ** 31, 2 ** 30, 131071, 65536, 4095,
                           123456789, -987654], np.int32)
    check_case(qk, inp, dtype, 128, 1e-6, 1e4, True, "extreme positions " + dtype)


def test_zero_tokens_is_a_noop(qk):
    z = torch.empty((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    zk = torch.empty((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    pos = torch.empty(0, dtype=torch.int32, device="cuda")
    yq, yk = qk.qknr_fwd(z, zk, w, w, pos, 64, 1e-6, 1e4)
    assert yq.shape == (0, 4, 64)
    dq, dk, dwq, dwk = qk.qknr_bwd(z, zk, w, w, pos, z, zk, 64, 1e-6, 1e4)
    torch.cuda.synchronize()
    assert dq.shape == (0, 4, 64)


def test_determinism_and_in_place(qk):
    """Two runs are bit-identical (dw included); in-place forward and backward
    give the same bits as out-of-place."""
    w = configs.QWEN05
    inp = gen.make_inputs(w, 0, 5000)
    d = dev_inputs(inp, w.dtype)
    args = (w.rotary_dim, w.eps, w.theta)
    a = qk.qknr_fwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], *args)
    b = qk.qknr_fwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], *args)
    ga = qk.qknr_bwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], d["dyq"], d["dyk"], *args)
    gb = qk.qknr_bwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], d["dyq"], d["dyk"], *args)
    for x, y in zip(a + ga, b + gb):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    qc, kc = d["q"].clone(), d["k"].clone()
    qk.qknr_fwd(qc, kc, d["wq"], d["wk"], d["pos"], *args, q_out=qc, k_out=kc)
    assert torch.equal(qc.view(torch.int16), a[0].view(torch.int16))
    assert torch.equal(kc.view(torch.int16), a[1].view(torch.int16))
    dyq, dyk = d["dyq"].clone(), d["dyk"].clone()
    r = qk.qknr_bwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], dyq, dyk, *args, dq=dyq, dk=dyk)
    torch.cuda.synchronize()
    for x, y in zip(r, ga):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_packed_documents_match_documents_alone(qk):
    """Packed buffer (BFD, positions restart per document): each document's rows
    are bit-identical to the document run alone (bf16 storage).  The weight
    gradient of the buffer equals the sum of the documents' weight gradients
    within fp32 reduction error, checked with fp32 storage so that no output
    rounding enters: the buffer's dw and the sum of the documents' dw each match
    the oracle's fp64 sum over every row within the fp32 rule for weight
    gradients (2e-5 * max(1, RMS)), and the two differ by at most twice that
    (a dropped or doubled row would move dw by about one row's g xh, far more)."""
    w = configs.PACKED
    pos, cu = gen.packed_layout(w)
    assert len(cu) - 1 >= 8   # the whole buffer: every document it packs
    inp = gen.make_inputs(w)
    d = dev_inputs(inp, w.dtype)
    args = (w.rotary_dim, w.eps, w.theta)
    yq, yk = qk.qknr_fwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], *args)
    dq, dk, _, _ = qk.qknr_bwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], d["dyq"], d["dyk"], *args)
    # fp32 copies of the same stored values for the weight-gradient identity
    f = {key: (t.float() if key != "pos" else t) for key, t in d.items()}
    _, _, fwq, fwk = qk.qknr_bwd(f["q"], f["k"], f["wq"], f["wk"], f["pos"], f["dyq"], f["dyk"],
                                 *args)
    sq = torch.zeros(w.head_dim, dtype=torch.float64, device="cuda")
    sk = torch.zeros_like(sq)
    for a, b in zip(cu[:-1], cu[1:]):
        sl = slice(int(a), int(b))
        p = torch.arange(int(b - a), dtype=torch.int32, device="cuda")
        assert torch.equal(d["pos"][sl], p)
        y1, y2 = qk.qknr_fwd(d["q"][sl].contiguous(), d["k"][sl].contiguous(), d["wq"], d["wk"], p, *args)
        g = qk.qknr_bwd(d["q"][sl].contiguous(), d["k"][sl].contiguous(), d["wq"], d["wk"], p,
                        d["dyq"][sl].contiguous(), d["dyk"][sl].contiguous(), *args)
        for x, y in ((y1, yq[sl]), (y2, yk[sl]), (g[0], dq[sl]), (g[1], dk[sl])):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16))
        gf = qk.qknr_bwd(f["q"][sl].contiguous(), f["k"][sl].contiguous(), f["wq"], f["wk"], p,
                         f["dyq"][sl].contiguous(), f["dyk"][sl].contiguous(), *args)
        sq += gf[2].double()
        sk += gf[3].double()
    torch.cuda.synchronize()
    o = run_oracle(inp, w.dtype, *args, True)
    for what, got, docs, ref in (("dwq", fwq, sq, o["dwq"]), ("dwk", fwk, sk, o["dwk"])):
        got = got.double().cpu().numpy()
        docs = docs.cpu().numpy()
        st_a = compare(got, ref, "f32", "packed fp32 " + what, row_sum=True)
        st_b = compare(docs, ref, "f32", "documents fp32 " + what, row_sum=True)
        err = float(np.abs(got - docs).max())
        say(what, "%d documents: buffer vs oracle %.3g, documents vs oracle %.3g, buffer vs "
            "documents %.3g, bound %.3g" % (len(cu) - 1, st_a["max_abs"], st_b["max_abs"], err,
                                           2 * st_a["tol"]))
        assert err <= 2 * st_a["tol"]


def test_head_and_token_permutations(qk):
    """Permuting heads, or tokens together with their positions, permutes the
    outputs bit for bit (row results do not depend on where a row sits)."""
    inp = gen.random_case(seed=5, tokens=97, hq=6, hkv=2, head_dim=64, dtype="bf16", max_pos=5000)
    d = dev_inputs(inp, "bf16")
    args = (64, 1e-6, 1e6)
    yq, yk = qk.qknr_fwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], *args)
    dq, dk, _, _ = qk.qknr_bwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], d["dyq"], d["dyk"], *args)
    hp = torch.tensor([3, 0, 5, 1, 4, 2], device="cuda")
    tp = torch.from_numpy(np.random.default_rng(1).permutation(97)).cuda()
    q2 = d["q"][tp][:, hp].contiguous()
    k2 = d["k"][tp].contiguous()
    y2q, y2k = qk.qknr_fwd(q2, k2, d["wq"], d["wk"], d["pos"][tp].contiguous(), *args)
    g2 = qk.qknr_bwd(q2, k2, d["wq"], d["wk"], d["pos"][tp].contiguous(),
                     d["dyq"][tp][:, hp].contiguous(), d["dyk"][tp].contiguous(), *args)
    torch.cuda.synchronize()
    assert torch.equal(y2q.view(torch.int16), yq[tp][:, hp].view(torch.int16))
    assert torch.equal(y2k.view(torch.int16), yk[tp].view(torch.int16))
    assert torch.equal(g2[0].view(torch.int16), dq[tp][:, hp].view(torch.int16))
    assert torch.equal(g2[1].view(torch.int16), dk[tp].view(torch.int16))


def test_binding_errors(qk):
    q = torch.zeros((4, 2, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(qk.QknrError) as e:
        qk.qknr_fwd(q, q, w, w, pos, 24, 1e-6, 1e4)
    assert e.value.status == 2
    small = torch.empty(8, dtype=torch.uint8, device="cuda")
    with pytest.raises(qk.QknrError) as e:
        qk.qknr_bwd(q, q, w, w, pos, q, q, 64, 1e-6, 1e4, workspace=small)
    assert e.value.status == 4
    with pytest.raises(TypeError):
        qk.qknr_fwd(q.half(), q.half(), w.half(), w.half(), pos, 64, 1e-6, 1e4)


def test_copy_and_flush_helpers(qk):
    from qk_norm_rope_amd import bench_helpers as bh
    src = torch.arange(1 << 20, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    bh.copy(src, dst)
    buf = torch.empty(1 << 16, dtype=torch.int32, device="cuda")
    bh.flush(buf, seed=3)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    assert int(buf[4]) == (1 ^ 3)  # element 4 is word 0 of 16-byte chunk 1
    # two reads, one write; a ragged count of 16-byte chunks
    a = torch.randint(-2**31, 2**31 - 1, (3 * 4096 + 12,), dtype=torch.int32, device="cuda")
    b = torch.randint(-2**31, 2**31 - 1, a.shape, dtype=torch.int32, device="cuda")
    c = torch.zeros_like(a)
    bh.stream2(a, b, c)
    torch.cuda.synchronize()
    assert torch.equal(c, a ^ b)

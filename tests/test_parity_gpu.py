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
from helpers import compare, gpu_values, to_device
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


def check_case(qk, inp, dtype, R, eps, theta, backward, what):
    say("case", what)
    g = run_gpu(qk, inp, dtype, R, eps, theta, backward)
    o = run_oracle(inp, dtype, R, eps, theta, backward)
    stats = {}
    for key in o:
        stats[key] = compare(gpu_values(g[key], dtype), o[key], dtype, "%s:%s" % (what, key),
                             row_sum=key.startswith("dw"))
    if backward:
        for key in ("dq", "dk", "dwq", "dwk"):  # gradients are really there (non-zero)
            assert np.abs(o[key]).max() > 1e-3 and np.abs(gpu_values(g[key], dtype)).max() > 1e-3
    return stats


def test_tiny_config(qk):
    w = configs.TINY
    inp = gen.make_inputs(w)
    st = check_case(qk, inp, w.dtype, w.rotary_dim, w.eps, w.theta, True, "tiny")
    say(st)


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


SWEEP = []
for _dt in ("f32", "bf16"):
    for _D in (64, 128, 256):
        for _R in sorted({0, 16, 32, _D // 2, _D}):
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


def _sample_tokens(T, n, seed):
    g = np.random.default_rng(seed)
    edge = np.concatenate([np.arange(0, 40), np.arange(T - 40, T),
                           np.arange(16, T, max(16, T // 64))[:64]])
    return np.unique(np.concatenate([g.choice(T, size=n, replace=False), edge]))


def test_full_config_7b_sampled_tokens_and_full_dw(qk):
    """7B-shaped configuration at full size: the GPU runs every row; outputs are
    compared on ~2.2k sampled tokens (all heads), dw against the oracle summed
    over every row."""
    w = configs.LLAMA7B
    say("generating", w.name)
    inp = gen.make_inputs(w)
    d = dev_inputs(inp, w.dtype)
    say("gpu", w.name)
    yq, yk = qk.qknr_fwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], w.rotary_dim, w.eps, w.theta)
    dq, dk, dwq, dwk = qk.qknr_bwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], d["dyq"], d["dyk"],
                                   w.rotary_dim, w.eps, w.theta)
    torch.cuda.synchronize()
    idx = _sample_tokens(w.tokens, 2048, 7)
    it = torch.from_numpy(idx).cuda()
    sub = {kk: inp[kk][idx] for kk in ("q", "k", "pos", "dyq", "dyk")}
    sub["wq"], sub["wk"] = inp["wq"], inp["wk"]
    say("oracle sample", w.name)
    o = run_oracle(sub, w.dtype, w.rotary_dim, w.eps, w.theta, True)
    for key, t in (("yq", yq), ("yk", yk), ("dq", dq), ("dk", dk)):
        compare(gpu_values(t.index_select(0, it), w.dtype), o[key], w.dtype, "7b:" + key)
    say("oracle dw over all rows", w.name)
    dec = lambda a: oracle.decode(a, w.dtype)  # noqa: E731
    owq = np.zeros(w.head_dim)
    owk = np.zeros(w.head_dim)
    for a in range(0, w.tokens, 4096):
        b = min(w.tokens, a + 4096)
        r = oracle.bwd(dec(inp["q"][a:b]), dec(inp["k"][a:b]), dec(inp["wq"]), dec(inp["wk"]),
                       inp["pos"][a:b], dec(inp["dyq"][a:b]), dec(inp["dyk"][a:b]), w.rotary_dim,
                       w.eps, w.theta, threads=THREADS)
        owq += r[2]
        owk += r[3]
    compare(gpu_values(dwq, w.dtype), owq, w.dtype, "7b:dwq", row_sum=True)
    compare(gpu_values(dwk, w.dtype), owk, w.dtype, "7b:dwk", row_sum=True)


def test_full_config_long_forward_sampled(qk):
    """Long-context partial-RoPE forward (131072 tokens, 72 heads, D=128, R=32)
    at full size; outputs compared on ~2.2k sampled tokens, including the
    largest positions."""
    w = configs.LONG
    say("generating", w.name)
    inp = gen.make_inputs(w, backward=False)
    d = dev_inputs(inp, w.dtype)
    say("gpu", w.name)
    yq, yk = qk.qknr_fwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], w.rotary_dim, w.eps, w.theta)
    torch.cuda.synchronize()
    idx = _sample_tokens(w.tokens, 2048, 8)
    it = torch.from_numpy(idx).cuda()
    sub = {kk: inp[kk][idx] for kk in ("q", "k", "pos")}
    sub["wq"], sub["wk"] = inp["wq"], inp["wk"]
    o = run_oracle(sub, w.dtype, w.rotary_dim, w.eps, w.theta, False)
    for key, t in (("yq", yq), ("yk", yk)):
        compare(gpu_values(t.index_select(0, it), w.dtype), o[key], w.dtype, "long:" + key)


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
    are bit-identical to the document run alone; dw of the buffer equals the sum
    of the documents' dw within the bf16 rule."""
    w = configs.PACKED
    pos, cu = gen.packed_layout(w)
    T = 6000
    cu = cu[cu <= T]
    inp = gen.make_inputs(w, 0, int(cu[-1]))
    d = dev_inputs(inp, w.dtype)
    args = (w.rotary_dim, w.eps, w.theta)
    yq, yk = qk.qknr_fwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], *args)
    dq, dk, dwq, dwk = qk.qknr_bwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], d["dyq"], d["dyk"], *args)
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
        sq += g[2].double()
        sk += g[3].double()
    torch.cuda.synchronize()
    # the per-document dw are themselves bf16-rounded, so allow their rounding too
    for got, ref in ((dwq, sq), (dwk, sk)):
        got = got.double().cpu().numpy()
        ref = ref.cpu().numpy()
        tol = 2.0 ** -6 * np.abs(ref).max() + (len(cu) - 1) * 2.0 ** -8 * np.abs(ref).max()
        assert np.abs(got - ref).max() <= tol


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
    src = torch.arange(1 << 20, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    qk.qknr_copy(src, dst)
    buf = torch.empty(1 << 16, dtype=torch.int32, device="cuda")
    qk.qknr_flush(buf, seed=3)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    assert int(buf[4]) == (1 ^ 3)  # element 4 is word 0 of 16-byte chunk 1
    # two reads, one write; a ragged count of 16-byte chunks
    a = torch.randint(-2**31, 2**31 - 1, (3 * 4096 + 12,), dtype=torch.int32, device="cuda")
    b = torch.randint(-2**31, 2**31 - 1, a.shape, dtype=torch.int32, device="cuda")
    c = torch.zeros_like(a)
    qk.qknr_stream2(a, b, c)
    torch.cuda.synchronize()
    assert torch.equal(c, a ^ b)

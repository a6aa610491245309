"""Parity of the extended entry points (qknr_fwd_ex / qknr_bwd_ex) with the
fp64 oracle: strided views of a fused QKV buffer written in place, the
convention flags (interleaved pairs, frequencies over the head width,
parameter-free norm), and K written through a slot map into a paged cache at
decode shapes.  Same tolerance rules as the dense path (helpers.py); bytes the
call must not touch are checked bit for bit.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from helpers import compare, gpu_values, to_device, to_host_bits
from workloads import gen

pytestmark = pytest.mark.gpu

try:
    THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
except AttributeError:  # pragma: no cover
    THREADS = 4

IL, FH, NW = 1, 2, 4   # QKNR_FLAG_INTERLEAVED, _FREQ_HEAD_DIM, _NO_WEIGHT


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def qk():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import qk_norm_rope_amd
    torch.cuda.set_device(0)
    return qk_norm_rope_amd


def oracle_flags(flags):
    return oracle.flags_of(interleaved=bool(flags & IL), freq_head_dim=bool(flags & FH))


def oracle_ref(inp, dtype, R, eps, theta, flags, backward):
    dec = lambda a: oracle.decode(a, dtype)  # noqa: E731
    q, k = dec(inp["q"]), dec(inp["k"])
    D = q.shape[2]
    if flags & NW:
        wq = wk = np.ones(D)
    else:
        wq, wk = dec(inp["wq"]), dec(inp["wk"])
    of = oracle_flags(flags)
    yq, yk = oracle.fwd(q, k, wq, wk, inp["pos"], R, eps, theta, threads=THREADS, flags=of)
    out = {"yq": yq, "yk": yk}
    if backward:
        dq, dk, dwq, dwk = oracle.bwd(q, k, wq, wk, inp["pos"], dec(inp["dyq"]), dec(inp["dyk"]),
                                      R, eps, theta, threads=THREADS, flags=of)
        out.update(dq=dq, dk=dk, dwq=dwq, dwk=dwk)
    return out


def fused(parts, dtype, pad, seed):
    """Concatenate [T, H_i, D] stored arrays along heads into one [T, W] buffer
    with `pad` extra elements of noise per token; returns (host array,
    element offsets of the parts)."""
    T = parts[0].shape[0]
    widths = [p.shape[1] * p.shape[2] for p in parts]
    g = np.random.default_rng(seed)
    noise = gen.encode(g.standard_normal((T, pad)), dtype) if pad else None
    cols = [p.reshape(T, -1) for p in parts] + ([noise] if pad else [])
    offs = np.cumsum([0] + widths)[:-1]
    return np.concatenate(cols, axis=1), [int(o) for o in offs]


def view3(buf, off, heads, D):
    return buf[:, off: off + heads * D].unflatten(1, (heads, D))


CASES = [  # dtype, D, R, T, hq, hkv, pad (elements of padding per token)
    ("bf16", 64, 64, 307, 14, 2, 0),
    ("bf16", 128, 64, 203, 8, 8, 8),
    ("bf16", 256, 128, 65, 3, 1, 24),
    ("f32", 64, 32, 150, 14, 2, 4),
    ("f32", 128, 128, 97, 5, 3, 0),
    ("f32", 256, 256, 33, 2, 2, 12),
]


@pytest.mark.parametrize("dtype,D,R,T,hq,hkv,pad", CASES)
def test_fused_qkv_in_place_forward(qk, dtype, D, R, T, hq, hkv, pad):
    """Q and K are views of one [T, (hq + 2 hkv) D (+ pad)] projection output;
    the kernel rotates them in place and leaves V and the padding alone."""
    what = "fused fwd %s D=%d R=%d T=%d hq=%d hkv=%d pad=%d" % (dtype, D, R, T, hq, hkv, pad)
    inp = gen.random_case(seed=7 * D + R + T, tokens=T, hq=hq, hkv=hkv, head_dim=D, dtype=dtype,
                          scale=1.3, max_pos=300000, backward=False)
    v = gen.encode(np.random.default_rng(T).standard_normal((T, hkv, D)), dtype)
    host, (oq, ok, ov) = fused([inp["q"], inp["k"], v], dtype, pad, seed=D)
    say("case", what)
    buf = to_device(host, dtype)
    q, k = view3(buf, oq, hq, D), view3(buf, ok, hkv, D)
    wq, wk = to_device(inp["wq"], dtype), to_device(inp["wk"], dtype)
    pos = torch.from_numpy(inp["pos"]).cuda()
    qk.qknr_fwd_ex(q, k, wq, wk, pos, R, 1e-6, 1e6, q_out=q, k_out=k)
    torch.cuda.synchronize()
    o = oracle_ref(inp, dtype, R, 1e-6, 1e6, 0, False)
    compare(gpu_values(q, dtype), o["yq"], dtype, what + ":yq")
    compare(gpu_values(k, dtype), o["yk"], dtype, what + ":yk")
    after = to_host_bits(buf, dtype)
    assert np.array_equal(after[:, ov:], host[:, ov:]), "V or padding was modified"


@pytest.mark.parametrize("dtype,D,R,T,hq,hkv,pad", CASES)
def test_fused_qkv_backward_in_place(qk, dtype, D, R, T, hq, hkv, pad):
    """Inputs and upstream gradients are views of fused buffers; dq/dk
    overwrite dq_out/dk_out in place; the dV slice and padding stay put."""
    what = "fused bwd %s D=%d R=%d T=%d hq=%d hkv=%d pad=%d" % (dtype, D, R, T, hq, hkv, pad)
    inp = gen.random_case(seed=11 * D + R + T, tokens=T, hq=hq, hkv=hkv, head_dim=D, dtype=dtype,
                          scale=0.9, max_pos=70000, backward=True)
    v = gen.encode(np.random.default_rng(T + 1).standard_normal((T, hkv, D)), dtype)
    hx, (oq, ok, _) = fused([inp["q"], inp["k"], v], dtype, pad, seed=D + 1)
    hg, (gq, gk, gv) = fused([inp["dyq"], inp["dyk"], v], dtype, pad, seed=D + 2)
    say("case", what)
    bx, bg = to_device(hx, dtype), to_device(hg, dtype)
    q, k = view3(bx, oq, hq, D), view3(bx, ok, hkv, D)
    dyq, dyk = view3(bg, gq, hq, D), view3(bg, gk, hkv, D)
    wq, wk = to_device(inp["wq"], dtype), to_device(inp["wk"], dtype)
    pos = torch.from_numpy(inp["pos"]).cuda()
    dq, dk, dwq, dwk = qk.qknr_bwd_ex(q, k, wq, wk, pos, dyq, dyk, R, 1e-6, 1e6, dq=dyq, dk=dyk)
    torch.cuda.synchronize()
    o = oracle_ref(inp, dtype, R, 1e-6, 1e6, 0, True)
    for key, t in (("dq", dq), ("dk", dk), ("dwq", dwq), ("dwk", dwk)):
        compare(gpu_values(t, dtype), o[key], dtype, what + ":" + key, row_sum=key.startswith("dw"))
    assert np.array_equal(to_host_bits(bg, dtype)[:, gv:], hg[:, gv:]), "dV or padding modified"
    assert np.array_equal(to_host_bits(bx, dtype), hx), "inputs modified"


FLAG_SETS = [IL, FH, NW, IL | FH, IL | NW, IL | FH | NW]


@pytest.mark.parametrize("flags", FLAG_SETS)
@pytest.mark.parametrize("dtype,D,R", [("bf16", 64, 64), ("bf16", 128, 32), ("f32", 128, 64),
                                       ("f32", 256, 256), ("bf16", 256, 16)])
def test_flags_forward_backward(qk, flags, dtype, D, R):
    T, hq, hkv = 123, 6, 2
    what = "flags=%d %s D=%d R=%d" % (flags, dtype, D, R)
    inp = gen.random_case(seed=flags * 100 + D + R, tokens=T, hq=hq, hkv=hkv, head_dim=D,
                          dtype=dtype, scale=1.1, max_pos=500000, backward=True)
    say("case", what)
    d = {key: to_device(val, dtype) for key, val in inp.items() if key != "pos"}
    pos = torch.from_numpy(inp["pos"]).cuda()
    wq, wk = (None, None) if flags & NW else (d["wq"], d["wk"])
    yq, yk = qk.qknr_fwd_ex(d["q"], d["k"], wq, wk, pos, R, 1e-5, 1e4, flags=flags)
    dq, dk, dwq, dwk = qk.qknr_bwd_ex(d["q"], d["k"], wq, wk, pos, d["dyq"], d["dyk"], R, 1e-5,
                                      1e4, flags=flags)
    torch.cuda.synchronize()
    o = oracle_ref(inp, dtype, R, 1e-5, 1e4, flags, True)
    for key, t in (("yq", yq), ("yk", yk), ("dq", dq), ("dk", dk)):
        compare(gpu_values(t, dtype), o[key], dtype, what + ":" + key)
    if flags & NW:
        assert dwq is None and dwk is None
    else:
        compare(gpu_values(dwq, dtype), o["dwq"], dtype, what + ":dwq", row_sum=True)
        compare(gpu_values(dwk, dtype), o["dwk"], dtype, what + ":dwk", row_sum=True)
    if R < D and (flags & FH):
        # the flag changes the frequencies: the default result differs
        dflt = oracle_ref(inp, dtype, R, 1e-5, 1e4, flags & ~FH, False)
        assert np.abs(dflt["yq"] - o["yq"]).max() > 1e-2


def test_no_weight_leaves_dw_buffers_alone(qk):
    """With the parameter-free flag the backward writes no weight gradient,
    even when buffers are passed."""
    T, hq, hkv, D, R = 40, 4, 2, 128, 64
    inp = gen.random_case(seed=5, tokens=T, hq=hq, hkv=hkv, head_dim=D, dtype="bf16",
                          max_pos=1000, backward=True)
    say("case no-weight dw untouched")
    d = {key: to_device(val, "bf16") for key, val in inp.items() if key != "pos"}
    pos = torch.from_numpy(inp["pos"]).cuda()
    sentinel = torch.full((D,), 3.0, dtype=torch.bfloat16, device="cuda")
    dwq, dwk = sentinel.clone(), sentinel.clone()
    lib = qk.lib
    import ctypes
    lay = qk.QknrLayout(hq * D, hkv * D, hq * D, hkv * D, hq * D, hkv * D, None, 0)
    dq, dk = torch.empty_like(d["q"]), torch.empty_like(d["k"])
    ws = torch.empty(qk.qknr_bwd_workspace_bytes(T, hq, hkv, D, qk.QKNR_BF16), dtype=torch.uint8,
                     device="cuda")
    st = lib.qknr_bwd_ex(d["q"].data_ptr(), d["k"].data_ptr(), None, None, pos.data_ptr(), T, hq,
                         hkv, D, R, 1e-5, 1e4, qk.QKNR_BF16, NW, ctypes.byref(lay),
                         d["dyq"].data_ptr(), d["dyk"].data_ptr(), dq.data_ptr(), dk.data_ptr(),
                         dwq.data_ptr(), dwk.data_ptr(), ws.data_ptr(), ws.numel(),
                         torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert torch.equal(dwq, sentinel) and torch.equal(dwk, sentinel)
    o = oracle_ref(inp, "bf16", R, 1e-5, 1e4, NW, True)
    compare(gpu_values(dq, "bf16"), o["dq"], "bf16", "no-weight dq")


DECODE = [  # dtype, batch (tokens), hq, hkv, D, R, cache slots
    ("bf16", 64, 14, 2, 64, 64, 4096),
    ("bf16", 256, 32, 8, 128, 128, 16384),
    ("bf16", 1, 32, 32, 128, 128, 512),
    ("f32", 37, 8, 1, 256, 64, 1000),
]


@pytest.mark.parametrize("dtype,B,hq,hkv,D,R,nslots", DECODE)
def test_decode_paged_k(qk, dtype, B, hq, hkv, D, R, nslots):
    """A decode step: one new token per sequence at a long-context position
    (up to 256k), Q written densely, K written into a paged cache
    [blocks * block_size, hkv, D] at each token's slot; slot -1 (padding) writes
    nothing, and every other cache row keeps its bytes."""
    what = "decode %s B=%d hq=%d hkv=%d D=%d R=%d slots=%d" % (dtype, B, hq, hkv, D, R, nslots)
    inp = gen.random_case(seed=B + hq + D, tokens=B, hq=hq, hkv=hkv, head_dim=D, dtype=dtype,
                          scale=1.0, max_pos=262144, backward=False)
    g = np.random.default_rng(B * 7 + D)
    slots = g.permutation(nslots)[:B].astype(np.int64)
    if B > 2:
        slots[g.choice(B, size=max(1, B // 8), replace=False)] = -1
    cache_host = gen.encode(g.standard_normal((nslots, hkv, D)), dtype)
    say("case", what)
    cache = to_device(cache_host, dtype)
    d = {key: to_device(val, dtype) for key, val in inp.items() if key != "pos"}
    pos = torch.from_numpy(inp["pos"]).cuda()
    sl = torch.from_numpy(slots).cuda()
    yq, kc = qk.qknr_fwd_ex(d["q"], d["k"], d["wq"], d["wk"], pos, R, 1e-6, 1e6, k_out=cache,
                            k_out_slots=sl)
    torch.cuda.synchronize()
    assert kc.data_ptr() == cache.data_ptr()
    o = oracle_ref(inp, dtype, R, 1e-6, 1e6, 0, False)
    compare(gpu_values(yq, dtype), o["yq"], dtype, what + ":yq")
    after = to_host_bits(cache, dtype)
    live = slots >= 0
    compare(oracle.decode(after[slots[live]], dtype), o["yk"][live], dtype, what + ":cache")
    untouched = np.ones(nslots, bool)
    untouched[slots[live]] = False
    assert np.array_equal(after[untouched], cache_host[untouched]), "cache rows outside the slots changed"


def test_decode_slots_with_strided_cache_and_flags(qk):
    """Slot map into a cache whose rows carry padding (stride > hkv * D),
    together with interleaved pairs and Q taken from a fused buffer."""
    dtype, B, hq, hkv, D, R, nslots, pad = "bf16", 48, 16, 4, 128, 64, 300, 16
    inp = gen.random_case(seed=99, tokens=B, hq=hq, hkv=hkv, head_dim=D, dtype=dtype,
                          max_pos=200000, backward=False)
    g = np.random.default_rng(3)
    slots = g.permutation(nslots)[:B].astype(np.int64)
    cache_host = gen.encode(g.standard_normal((nslots, hkv * D + pad)), dtype)
    v = gen.encode(g.standard_normal((B, hkv, D)), dtype)
    host, (oq, ok, _) = fused([inp["q"], inp["k"], v], dtype, 0, seed=4)
    say("case decode strided cache + interleaved")
    buf, cache = to_device(host, dtype), to_device(cache_host, dtype)
    q, k = view3(buf, oq, hq, D), view3(buf, ok, hkv, D)
    kview = cache[:, : hkv * D].unflatten(1, (hkv, D))
    d = {key: to_device(inp[key], dtype) for key in ("wq", "wk")}
    pos = torch.from_numpy(inp["pos"]).cuda()
    yq, _ = qk.qknr_fwd_ex(q, k, d["wq"], d["wk"], pos, R, 1e-6, 1e4, flags=IL, q_out=q,
                           k_out=kview, k_out_slots=torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    o = oracle_ref(inp, dtype, R, 1e-6, 1e4, IL, False)
    compare(gpu_values(q, dtype), o["yq"], dtype, "strided decode yq")
    after = to_host_bits(cache, dtype)
    got_k = after[slots, : hkv * D].reshape(B, hkv, D)
    compare(oracle.decode(got_k, dtype), o["yk"], dtype, "strided decode cache")
    mask = np.ones(nslots, bool)
    mask[slots] = False
    assert np.array_equal(after[mask], cache_host[mask])
    assert np.array_equal(after[slots, hkv * D:], cache_host[slots, hkv * D:]), "row padding changed"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ex_dense_equals_plain_entry_points(qk, dtype):
    """With dense views and no flags the extended entry points run the same
    kernels: results are bit-identical to qknr_fwd / qknr_bwd."""
    T, hq, hkv, D, R = 211, 7, 1, 128, 64
    inp = gen.random_case(seed=1, tokens=T, hq=hq, hkv=hkv, head_dim=D, dtype=dtype,
                          max_pos=9000, backward=True)
    say("case ex == plain", dtype)
    d = {key: to_device(val, dtype) for key, val in inp.items() if key != "pos"}
    pos = torch.from_numpy(inp["pos"]).cuda()
    a = qk.qknr_fwd(d["q"], d["k"], d["wq"], d["wk"], pos, R, 1e-6, 1e4)
    b = qk.qknr_fwd_ex(d["q"], d["k"], d["wq"], d["wk"], pos, R, 1e-6, 1e4)
    ga = qk.qknr_bwd(d["q"], d["k"], d["wq"], d["wk"], pos, d["dyq"], d["dyk"], R, 1e-6, 1e4)
    gb = qk.qknr_bwd_ex(d["q"], d["k"], d["wq"], d["wk"], pos, d["dyq"], d["dyk"], R, 1e-6, 1e4)
    torch.cuda.synchronize()
    for x, y in zip(list(a) + list(ga), list(b) + list(gb)):
        assert torch.equal(x, y)


def test_binding_rejects_bad_views(qk):
    T, hq, hkv, D = 8, 2, 1, 64
    q = torch.zeros(T, hq, D, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(T, hkv, D, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(D, dtype=torch.bfloat16, device="cuda")
    pos = torch.zeros(T, dtype=torch.int32, device="cuda")
    say("case binding errors")
    with pytest.raises(ValueError):   # heads not contiguous
        qk.qknr_fwd_ex(q.transpose(0, 1).contiguous().transpose(0, 1), k, w, w, pos, 64, 1e-6, 1e4)
    with pytest.raises(qk.QknrError):   # token stride not a whole number of 16-byte chunks
        big = torch.zeros(T, hq * D + 4, dtype=torch.bfloat16, device="cuda")
        qk.qknr_fwd_ex(big[:, : hq * D].unflatten(1, (hq, D)), k, w, w, pos, 64, 1e-6, 1e4)
    with pytest.raises(ValueError):   # slots without the buffer they index
        qk.qknr_fwd_ex(q, k, w, w, pos, 64, 1e-6, 1e4,
                       k_out_slots=torch.zeros(T, dtype=torch.int64, device="cuda"))
    with pytest.raises(qk.QknrError):   # unknown flag bit
        qk.qknr_fwd_ex(q, k, w, w, pos, 64, 1e-6, 1e4, flags=64)


def test_graph_replays_equal_eager(qk):
    """The calls capture into a HIP graph (no allocation, no memset nodes): each
    replay, with eager work and a synchronisation between replays, reproduces
    the eager results bit for bit (forward, backward with dw, slot-mapped
    decode)."""
    dtype, T, hq, hkv, D, R = "bf16", 96, 8, 2, 128, 128
    inp = gen.random_case(seed=77, tokens=T, hq=hq, hkv=hkv, head_dim=D, dtype=dtype,
                          max_pos=100000, backward=True)
    say("case graph replay")
    d = {key: to_device(val, dtype) for key, val in inp.items() if key != "pos"}
    pos = torch.from_numpy(inp["pos"]).cuda()
    nslots = 1000
    slots = torch.from_numpy(np.random.default_rng(0).permutation(nslots)[:T].astype(np.int64)).cuda()
    outs = dict(yq=torch.empty_like(d["q"]), yk=torch.empty_like(d["k"]),
                dq=torch.empty_like(d["q"]), dk=torch.empty_like(d["k"]),
                dwq=torch.empty_like(d["wq"]), dwk=torch.empty_like(d["wk"]),
                dec_q=torch.empty_like(d["q"]),
                cache=torch.zeros(nslots, hkv, D, dtype=torch.bfloat16, device="cuda"))
    ws = torch.empty(qk.qknr_bwd_workspace_bytes(T, hq, hkv, D, qk.QKNR_BF16), dtype=torch.uint8,
                     device="cuda")

    def calls():
        qk.qknr_fwd(d["q"], d["k"], d["wq"], d["wk"], pos, R, 1e-6, 1e4, q_out=outs["yq"],
                    k_out=outs["yk"])
        qk.qknr_bwd(d["q"], d["k"], d["wq"], d["wk"], pos, d["dyq"], d["dyk"], R, 1e-6, 1e4,
                    dq=outs["dq"], dk=outs["dk"], dwq=outs["dwq"], dwk=outs["dwk"], workspace=ws)
        qk.qknr_fwd_ex(d["q"], d["k"], d["wq"], d["wk"], pos, R, 1e-6, 1e4, q_out=outs["dec_q"],
                       k_out=outs["cache"], k_out_slots=slots)

    calls()
    torch.cuda.synchronize()
    eager = {key: t.clone() for key, t in outs.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(4):
        for t in outs.values():
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key, t in outs.items():
            assert torch.equal(t, eager[key]), "replay %d differs in %s" % (rep, key)
    o = oracle_ref(inp, dtype, R, 1e-6, 1e4, 0, True)
    compare(gpu_values(outs["yq"], dtype), o["yq"], dtype, "graph yq")
    compare(gpu_values(outs["dwq"], dtype), o["dwq"], dtype, "graph dwq", row_sum=True)


@pytest.mark.parametrize("mode", ["plain", "interleaved", "layernorm_bias_table"])
def test_split_forward_matches_dense(qk, mode):
    """Forwards of at most 1024 tokens whose rows span several wave stages (here
    7B-shaped heads: 40 rows of 128 over five stages) give each stage of a token
    its own wave, through the norm-group wave kernel with groups of one head.
    Its arithmetic is the dense kernel's, so the first 1024 tokens of a
    1025-token call (the dense kernel) and the same 1024 tokens alone (split)
    agree bit for bit; the split call also matches the oracle."""
    dtype, hq, hkv, D, R, T = "bf16", 32, 8, 128, 128, 1025
    inp = gen.random_case(seed=31, tokens=T, hq=hq, hkv=hkv, head_dim=D, dtype=dtype,
                          max_pos=262144, backward=False)
    d = {key: to_device(val, dtype) for key, val in inp.items() if key != "pos"}
    pos = torch.from_numpy(inp["pos"]).cuda()
    g = np.random.default_rng(32)
    bq = to_device(gen.encode(0.1 * g.standard_normal(D), dtype), dtype)
    bk = to_device(gen.encode(0.1 * g.standard_normal(D), dtype), dtype)
    table = [5e5 ** (-2.0 * i / R) / 4.0 for i in range(R // 2)]
    say("case split forward", mode)

    def run(n):
        q, k, p = d["q"][:n].contiguous(), d["k"][:n].contiguous(), pos[:n].contiguous()
        if mode == "plain":
            return qk.qknr_fwd(q, k, d["wq"], d["wk"], p, R, 1e-5, 5e5)
        if mode == "interleaved":
            return qk.qknr_fwd_ex(q, k, d["wq"], d["wk"], p, R, 1e-5, 5e5, flags=IL)
        return qk.qknr_fwd_opt(q, k, d["wq"], d["wk"], p, R, 1e-5, 5e5, flags=8, bq=bq, bk=bk,
                               inv_freq=table, attention_factor=1.1)

    yq_all, yk_all = run(T)
    yq, yk = run(1024)
    torch.cuda.synchronize()
    assert torch.equal(yq_all[:1024].view(torch.int16), yq.view(torch.int16)), mode
    assert torch.equal(yk_all[:1024].view(torch.int16), yk.view(torch.int16)), mode
    if mode == "plain":
        sub = {key: val[:1024] for key, val in inp.items()}
        o = oracle_ref(sub, dtype, R, 1e-5, 5e5, 0, False)
        compare(gpu_values(yq, dtype), o["yq"], dtype, "split forward:yq")
        compare(gpu_values(yk, dtype), o["yk"], dtype, "split forward:yk")

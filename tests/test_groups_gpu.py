"""Parity of norm groups and per-head weights (qknr_fwd_opt / qknr_bwd_opt with
norm_group_q/k and QKNR_FLAG_HEAD_WEIGHTS, the whole-token kernel) with the fp64
oracle: groups of GQA size (one inverse RMS per token and head group, as in
QK-Normed MLA), the layerwise norm over a token's whole q / k vector, and [H, D]
weights, biases and their gradients, with the other options (LayerNorm,
interleaved pairs, parameter-free norm, frequency table, strided views).
Same tolerance rules as the dense path (helpers.py).
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

IL, FH, NW, LN, HW = 1, 2, 4, 8, 16   # library flag bits


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def qk():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import qk_norm_rope_amd
    torch.cuda.set_device(0)
    return qk_norm_rope_amd


def make_case(seed, T, hq, hkv, D, dtype, head_w, bias, max_pos=100000):
    inp = gen.random_case(seed=seed, tokens=T, hq=hq, hkv=hkv, head_dim=D, dtype=dtype,
                          scale=1.0, max_pos=max_pos, backward=True)
    g = np.random.default_rng(seed + 1)
    # per-head scales and offsets, so that a group's statistics differ from its heads'
    for key, H in (("q", hq), ("k", hkv)):
        x = oracle.decode(inp[key], dtype)
        x = x * (0.5 + g.random((1, H, 1))) + 0.3 * g.standard_normal((1, H, 1))
        inp[key] = gen.encode(x, dtype)
    if head_w:
        inp["wq"] = gen.encode(1 + 0.2 * g.standard_normal((hq, D)), dtype)
        inp["wk"] = gen.encode(1 + 0.2 * g.standard_normal((hkv, D)), dtype)
    if bias:
        shq, shk = ((hq, D), (hkv, D)) if head_w else ((D,), (D,))
        inp["bq"] = gen.encode(0.2 * g.standard_normal(shq), dtype)
        inp["bk"] = gen.encode(0.2 * g.standard_normal(shk), dtype)
    return inp


def oracle_ref(inp, dtype, R, eps, theta, flags, groups, bias, table=None):
    dec = lambda a: oracle.decode(a, dtype)  # noqa: E731
    q, k = dec(inp["q"]), dec(inp["k"])
    hq, hkv, D = q.shape[1], k.shape[1], q.shape[2]
    head_w = bool(flags & HW)
    if flags & NW:
        wq, wk = (np.ones((hq, D)), np.ones((hkv, D))) if head_w else (np.ones(D), np.ones(D))
    else:
        wq, wk = dec(inp["wq"]), dec(inp["wk"])
    of = oracle.flags_of(interleaved=bool(flags & IL), freq_head_dim=bool(flags & FH),
                         layernorm=bool(flags & LN), head_weights=head_w)
    bq, bk = (dec(inp["bq"]), dec(inp["bk"])) if bias else (None, None)
    yq, yk = oracle.fwd(q, k, wq, wk, inp["pos"], R, eps, theta, threads=THREADS, flags=of,
                        bq=bq, bk=bk, inv_freq=table, norm_groups=groups)
    r = oracle.bwd(q, k, wq, wk, inp["pos"], dec(inp["dyq"]), dec(inp["dyk"]), R, eps, theta,
                   threads=THREADS, flags=of, inv_freq=table, bias_grads=bias, norm_groups=groups)
    out = {"yq": yq, "yk": yk}
    out.update(zip(("dq", "dk", "dwq", "dwk", "dbq", "dbk"), r))
    return out


def run_case(qk, inp, dtype, R, eps, theta, flags, groups, bias, table=None, what=""):
    d = {key: to_device(val, dtype) for key, val in inp.items() if key != "pos"}
    pos = torch.from_numpy(inp["pos"]).cuda()
    wq, wk = (None, None) if flags & NW else (d["wq"], d["wk"])
    bq, bk = (d["bq"], d["bk"]) if bias else (None, None)
    yq, yk = qk.qknr_fwd_opt(d["q"], d["k"], wq, wk, pos, R, eps, theta, flags=flags, bq=bq,
                             bk=bk, inv_freq=table, norm_groups=groups)
    grads = qk.qknr_bwd_opt(d["q"], d["k"], wq, wk, pos, d["dyq"], d["dyk"], R, eps, theta,
                            flags=flags, bias_grads=bias, inv_freq=table, norm_groups=groups)
    torch.cuda.synchronize()
    o = oracle_ref(inp, dtype, R, eps, theta, flags, groups, bias, table)
    got = dict(zip(("yq", "yk", "dq", "dk", "dwq", "dwk", "dbq", "dbk"), (yq, yk) + tuple(grads)))
    for key in ("yq", "yk", "dq", "dk"):
        compare(gpu_values(got[key], dtype), o[key], dtype, what + ":" + key)
    for key in ("dwq", "dwk", "dbq", "dbk"):
        want_none = (key.startswith("dw") and flags & NW) or (key.startswith("db") and not bias)
        if want_none:
            assert got[key] is None, key
        else:
            compare(gpu_values(got[key], dtype), o[key], dtype, what + ":" + key, row_sum=True)


GROUP_CASES = [  # dtype, D, R, T, hq, hkv, gq, gk
    ("bf16", 64, 64, 131, 14, 2, 7, 1),      # Qwen-shaped GQA groups for q, per head for k
    ("bf16", 64, 64, 97, 14, 2, 14, 2),      # layerwise: every head of q, every head of k
    ("bf16", 128, 128, 45, 32, 8, 4, 8),     # 7B-shaped: q in GQA groups, k layerwise
    ("bf16", 256, 64, 19, 4, 2, 2, 1),
    ("f32", 64, 32, 83, 6, 2, 3, 2),
    ("f32", 128, 128, 37, 8, 4, 8, 1),
    ("f32", 256, 256, 11, 2, 2, 2, 2),
    ("bf16", 128, 0, 1, 2, 6, 2, 3),         # no rotation, one token, more k heads than q heads
    ("f32", 64, 16, 5, 3, 3, 3, 1),          # the narrowest rotary width
    ("bf16", 64, 64, 97, 4, 2, 2, 1),        # two 6-row tokens per 16-row wave stage, ragged end
    ("bf16", 64, 32, 131, 6, 2, 3, 2),       # two 8-row tokens fill a stage, ragged end
    ("bf16", 64, 64, 57, 20, 2, 4, 2),       # a token over two 16-row stages, groups inside them
    ("bf16", 64, 64, 57, 20, 2, 5, 2),       # a q group across the stages: whole tokens
    ("bf16", 64, 64, 45, 14, 4, 7, 4),       # the k group across the stages: whole tokens
    ("bf16", 64, 64, 45, 14, 4, 7, 2),       # k groups inside the second stage
    ("bf16", 128, 128, 23, 32, 8, 32, 8),    # 7B-shaped layerwise: 32-row q group over four stages
    ("bf16", 64, 64, 13, 70, 2, 70, 1),      # a 70-row q group: more rows than a wave's lanes
]


@pytest.mark.parametrize("head_w,bias,flags", [(False, False, 0), (True, True, 0),
                                                (True, False, LN), (False, True, LN | IL)])
@pytest.mark.parametrize("dtype,D,R,T,hq,hkv,gq,gk", GROUP_CASES)
def test_norm_groups(qk, dtype, D, R, T, hq, hkv, gq, gk, head_w, bias, flags):
    flags = flags | (HW if head_w else 0)
    what = "groups %s D=%d R=%d T=%d hq=%d hkv=%d g=(%d,%d) flags=%d bias=%d" % (
        dtype, D, R, T, hq, hkv, gq, gk, flags, bias)
    inp = make_case(D + T + gq * 3 + flags, T, hq, hkv, D, dtype, head_w, bias)
    say("case", what)
    run_case(qk, inp, dtype, R, 1e-5, 1e6, flags, (gq, gk), bias, what=what)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_per_head_weights_groups_of_one(qk, dtype, D):
    """[H, D] weights with the per-head norm (groups of one), with a frequency
    table and no weights at all."""
    T, hq, hkv, R = 70, 6, 3, D // 2
    table = 1e4 ** (-2.0 * np.arange(R // 2) / R) / 3.0
    for flags, bias in ((HW, True), (HW | NW, False), (HW | FH, False)):
        what = "per-head weights %s D=%d flags=%d" % (dtype, D, flags)
        inp = make_case(D + flags, T, hq, hkv, D, dtype, True, bias)
        say("case", what)
        run_case(qk, inp, dtype, R, 1e-6, 1e4, flags, (1, 1), bias, table=table, what=what)


def test_groups_on_fused_views(qk):
    """Layerwise q norm and per-head k norm with [H, D] weights on Q/K views of
    a fused QKV buffer, rotated in place; V untouched."""
    dtype, T, hq, hkv, D, R = "bf16", 88, 8, 2, 128, 64
    inp = make_case(5, T, hq, hkv, D, dtype, True, True)
    v = gen.encode(np.random.default_rng(6).standard_normal((T, hkv, D)), dtype)
    host = np.concatenate([inp["q"].reshape(T, -1), inp["k"].reshape(T, -1), v.reshape(T, -1)], 1)
    say("case groups on fused views")
    buf = to_device(host, dtype)
    q = buf[:, : hq * D].unflatten(1, (hq, D))
    k = buf[:, hq * D: (hq + hkv) * D].unflatten(1, (hkv, D))
    d = {key: to_device(inp[key], dtype) for key in ("wq", "wk", "bq", "bk")}
    qk.qknr_fwd_opt(q, k, d["wq"], d["wk"], torch.from_numpy(inp["pos"]).cuda(), R, 1e-6, 1e6,
                    flags=HW, bq=d["bq"], bk=d["bk"], norm_groups=(hq, 1), q_out=q, k_out=k)
    torch.cuda.synchronize()
    o = oracle_ref(inp, dtype, R, 1e-6, 1e6, HW, (hq, 1), True)
    compare(gpu_values(q, dtype), o["yq"], dtype, "fused groups yq")
    compare(gpu_values(k, dtype), o["yk"], dtype, "fused groups yk")
    after = buf[:, (hq + hkv) * D:].cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(after, v.reshape(T, -1))


@pytest.mark.parametrize("hq,hkv,D,groups", [(14, 2, 64, (7, 2)), (32, 8, 128, (4, 8))])
def test_groups_deterministic(qk, hq, hkv, D, groups):
    """Two backward runs give bit-identical gradients (fixed-order sums)."""
    dtype, T, R = "bf16", 300, D
    inp = make_case(9, T, hq, hkv, D, dtype, True, True)
    say("case groups deterministic", hq, hkv, D)
    d = {key: to_device(val, dtype) for key, val in inp.items() if key != "pos"}
    pos = torch.from_numpy(inp["pos"]).cuda()
    runs = []
    for _ in range(2):
        runs.append(qk.qknr_bwd_opt(d["q"], d["k"], d["wq"], d["wk"], pos, d["dyq"], d["dyk"], R,
                                    1e-6, 1e6, flags=HW, bias_grads=True, norm_groups=groups))
    torch.cuda.synchronize()
    for a, b in zip(*runs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype,D,hq,hkv,B,groups,flags", [("bf16", 128, 32, 8, 37, (4, 8), 0),
                                                           ("bf16", 64, 14, 2, 256, (7, 2), 0),
                                                           ("f32", 128, 8, 4, 1, (2, 1), 0),
                                                           ("bf16", 256, 8, 2, 19, (8, 2), 0),
                                                           ("bf16", 64, 14, 2, 64, (7, 2), IL),
                                                           ("f32", 64, 6, 2, 9, (3, 2), LN | IL)])
def test_groups_decode_into_paged_cache(qk, dtype, D, hq, hkv, B, groups, flags):
    """Decode steps with norm groups and [H, D] weights: one new token per
    sequence at positions up to 256k, Q written densely, K through the slot map
    into a paged cache [slots, hkv, D]; padded tokens (slot -1) write nothing
    and every other cache row is left alone."""
    R, nslots = D, 4096
    what = "groups decode %s D=%d hq=%d hkv=%d B=%d groups=%s flags=%d" % (dtype, D, hq, hkv, B,
                                                                         groups, flags)
    inp = make_case(B + D, B, hq, hkv, D, dtype, True, True, max_pos=262144)
    g = np.random.default_rng(B + 7)
    slots = g.permutation(nslots)[:B].astype(np.int64)
    if B > 2:
        slots[g.choice(B, size=B // 4, replace=False)] = -1   # padding
    say("case", what)
    d = {key: to_device(val, dtype) for key, val in inp.items() if key != "pos"}
    pos = torch.from_numpy(inp["pos"]).cuda()
    fill = gen.encode(g.standard_normal((nslots, hkv, D)), dtype)
    cache = to_device(fill, dtype)
    yq, _ = qk.qknr_fwd_opt(d["q"], d["k"], d["wq"], d["wk"], pos, R, 1e-6, 1e6, flags=HW | flags,
                            bq=d["bq"], bk=d["bk"], norm_groups=groups, k_out=cache,
                            k_out_slots=torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    dec = lambda a: oracle.decode(a, dtype)  # noqa: E731
    oq, ok_ = oracle.fwd(dec(inp["q"]), dec(inp["k"]), dec(inp["wq"]), dec(inp["wk"]), inp["pos"],
                         R, 1e-6, 1e6, threads=THREADS,
                         flags=oracle.flags_of(head_weights=True, interleaved=bool(flags & IL),
                                               layernorm=bool(flags & LN)),
                         bq=dec(inp["bq"]), bk=dec(inp["bk"]), norm_groups=groups)
    compare(gpu_values(yq, dtype), oq, dtype, what + ":yq")
    got = gpu_values(cache, dtype)
    live = slots >= 0
    compare(got[slots[live]], ok_[live], dtype, what + ":cache rows")
    untouched = np.setdiff1d(np.arange(nslots), slots[live])
    assert np.array_equal(got[untouched], dec(fill)[untouched])


@pytest.mark.parametrize("hq,hkv,backward,gq", [(120, 8, False, 15), (88, 8, True, 11),
                                                (120, 8, False, 8), (88, 8, True, 8)])
def test_groups_at_the_token_size_limits(qk, hq, hkv, backward, gq):
    """A token exactly as large as the norm-group kernels take: 128 bf16 rows
    of 128 (32 KiB) in the forward, 96 rows (24 KiB) in the backward; q groups
    of 15 or 11 heads cross the 8-row wave stages (whole tokens per workgroup),
    groups of 8 do not (16 and 12 stages per token)."""
    dtype, D, R, T = "bf16", 128, 64, 7
    groups = (gq, hkv)
    what = "groups at the limit hq=%d hkv=%d backward=%d gq=%d" % (hq, hkv, backward, gq)
    inp = make_case(hq + 3, T, hq, hkv, D, dtype, True, True)
    say("case", what)
    if backward:
        run_case(qk, inp, dtype, R, 1e-5, 1e6, HW, groups, True, what=what)
        return
    d = {key: to_device(val, dtype) for key, val in inp.items() if key != "pos"}
    pos = torch.from_numpy(inp["pos"]).cuda()
    yq, yk = qk.qknr_fwd_opt(d["q"], d["k"], d["wq"], d["wk"], pos, R, 1e-5, 1e6, flags=HW,
                             bq=d["bq"], bk=d["bk"], norm_groups=groups)
    torch.cuda.synchronize()
    dec = lambda a: oracle.decode(a, dtype)  # noqa: E731
    oq, ok_ = oracle.fwd(dec(inp["q"]), dec(inp["k"]), dec(inp["wq"]), dec(inp["wk"]), inp["pos"],
                         R, 1e-5, 1e6, threads=THREADS, flags=oracle.flags_of(head_weights=True),
                         bq=dec(inp["bq"]), bk=dec(inp["bk"]), norm_groups=groups)
    compare(gpu_values(yq, dtype), oq, dtype, what + ":yq")
    compare(gpu_values(yk, dtype), ok_, dtype, what + ":yk")


@pytest.mark.parametrize("kernel,hq,hkv,groups", [("dense", 14, 2, None),
                                                  ("wave", 14, 2, (7, 2)),
                                                  ("whole-token", 20, 2, (5, 2))])
def test_slots_past_k_out_rows_are_skipped(qk, kernel, hq, hkv, groups):
    """A slot at or past k_out's row count writes nothing (like a negative
    slot), in each kernel that writes K through a slot map.  The cache handed
    over as k_out is the first nslots rows of a larger allocation, so the rows
    after it would show any write that crossed its end."""
    dtype, D, R, B, nslots, guard = "bf16", 64, 64, 48, 300, 64
    what = "slots past k_out %s hq=%d hkv=%d groups=%s" % (kernel, hq, hkv, groups)
    inp = make_case(hq * 3 + hkv, B, hq, hkv, D, dtype, groups is not None, groups is not None,
                    max_pos=262144)
    g = np.random.default_rng(hq + 11)
    slots = g.permutation(nslots)[:B].astype(np.int64)
    past = g.choice(B, size=B // 3, replace=False)
    slots[past] = nslots + g.integers(0, guard, size=past.size)   # past k_out's end
    slots[past[:2]] = nslots                                        # exactly at it
    say("case", what)
    d = {key: to_device(val, dtype) for key, val in inp.items() if key != "pos"}
    pos = torch.from_numpy(inp["pos"]).cuda()
    fill = gen.encode(g.standard_normal((nslots + guard, hkv, D)), dtype)
    whole = to_device(fill, dtype)
    cache = whole[:nslots]
    sl = torch.from_numpy(slots).cuda()
    dec = lambda a: oracle.decode(a, dtype)  # noqa: E731
    if groups is None:
        yq, _ = qk.qknr_fwd_ex(d["q"], d["k"], d["wq"], d["wk"], pos, R, 1e-6, 1e6, k_out=cache,
                               k_out_slots=sl)
        oq, ok_ = oracle.fwd(dec(inp["q"]), dec(inp["k"]), dec(inp["wq"]), dec(inp["wk"]),
                             inp["pos"], R, 1e-6, 1e6, threads=THREADS)
    else:
        yq, _ = qk.qknr_fwd_opt(d["q"], d["k"], d["wq"], d["wk"], pos, R, 1e-6, 1e6, flags=HW,
                                bq=d["bq"], bk=d["bk"], norm_groups=groups, k_out=cache,
                                k_out_slots=sl)
        oq, ok_ = oracle.fwd(dec(inp["q"]), dec(inp["k"]), dec(inp["wq"]), dec(inp["wk"]),
                             inp["pos"], R, 1e-6, 1e6, threads=THREADS,
                             flags=oracle.flags_of(head_weights=True), bq=dec(inp["bq"]),
                             bk=dec(inp["bk"]), norm_groups=groups)
    torch.cuda.synchronize()
    compare(gpu_values(yq, dtype), oq, dtype, what + ":yq")
    got = gpu_values(whole, dtype)
    live = slots < nslots
    compare(got[slots[live]], ok_[live], dtype, what + ":cache rows")
    untouched = np.setdiff1d(np.arange(nslots + guard), slots[live])
    assert np.array_equal(got[untouched], dec(fill)[untouched]), "rows outside the live slots changed"

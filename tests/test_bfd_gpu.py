"""The device Best-Fit-Decreasing packer (qknr_bfd_pack) against the C oracle,
bit for bit: document starts, position ids, cu_seqlens and counts, on random
length mixes (log-uniform as in the packed workload, uniform, many equal
lengths, half the documents one token past half the capacity), edge cases
(no documents, one, every document filling a bin, one token each), every
placement the launch picks (one wave for up to 64 bins; the whole workgroup
with 1, 2 or 4 bins per thread for up to 1024, 2048 and 4096; the single-wave
loop over LDS for capacities of 2^20 and more) filled past 1024 and 2048 bins,
both error statuses on each placement; and the packed workload's own buffer
(the fullest bin) reproduced from its drawn lengths.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import bfd as host_bfd
from workloads import configs, gen

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def qk():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import qk_norm_rope_amd
    torch.cuda.set_device(0)
    return qk_norm_rope_amd


def lengths_of(kind, seed, n, cap):
    g = np.random.default_rng(seed)
    if kind == "loguniform":
        lo = max(1, min(16, cap))
        return np.clip(np.rint(np.exp(g.uniform(np.log(lo), np.log(cap), n))), 1, cap).astype(np.int32)
    if kind == "ties":
        return g.choice([cap // 2, cap // 3 + 1, cap // 4, 1], size=n).astype(np.int32)
    if kind == "full":
        return np.full(n, cap, np.int32)
    if kind == "ones":
        return np.ones(n, np.int32)
    if kind == "halves":
        # n documents, half of them one token past half the capacity (each
        # opens a bin of its own), the rest shorter than half, shuffled
        big = np.full(n - n // 2, cap // 2 + 1, np.int64)
        small = g.integers(1, cap // 2, size=n // 2)
        return g.permutation(np.concatenate([big, small])).astype(np.int32)
    return g.integers(1, cap + 1, size=n).astype(np.int32)


def device_pack(qk, L, cap, max_bins, keep_positions_on_device=False):
    lt = torch.from_numpy(np.ascontiguousarray(L, np.int32)).cuda()
    r = qk.qknr_bfd_pack(lt, cap, max_bins)
    torch.cuda.synchronize()
    return {k: (v if keep_positions_on_device and k == "position_ids" else v.cpu().numpy())
            for k, v in r.items()}


CASES = [  # kind, seed, ndocs, capacity, max_bins
    ("loguniform", 1, 356, 32768, 64),
    ("loguniform", 2, 2000, 4096, 1024),
    ("uniform", 3, 777, 1000, 800),
    ("ties", 4, 1500, 96, 1500),
    ("full", 5, 40, 128, 40),
    ("ones", 6, 1000, 64, 20),
    ("uniform", 7, 1, 5, 1),
    ("uniform", 8, 0, 16, 3),
    ("loguniform", 9, 5000, 8192, 4096),
    ("uniform", 10, 200, 512, 128),          # the workgroup placement, one bin per thread
    ("ties", 11, 900, 256, 256),             # the same
    ("loguniform", 12, 60, 1 << 20, 16),     # capacity 2^20: the unpacked (fill, bin) minimum
    ("halves", 13, 2000, 1000, 1024),        # 1000 bins, one per thread
    ("halves", 14, 2400, 1000, 2048),        # 1200 bins, two per thread
    ("halves", 15, 4400, 700, 4096),         # 2200 bins, four per thread
    ("halves", 16, 4096, 4096, 2048),        # 2048 bins: every slot of two per thread used
    ("halves", 17, 150, 1 << 20, 100),       # capacity 2^20, more than 64 bins: the LDS loop
]


@pytest.mark.parametrize("kind,seed,n,cap,max_bins", CASES)
def test_bfd_matches_oracle(qk, kind, seed, n, cap, max_bins):
    L = lengths_of(kind, seed, n, cap)
    say("case bfd", kind, seed, n, cap, max_bins)
    got = device_pack(qk, L, cap, max_bins, keep_positions_on_device=True)
    want = oracle.bfd_pack(L, cap, max_bins)
    assert int(got["status"][0]) == want["status"] == 0
    nb, ns = int(got["counts"][0]), int(got["counts"][1])
    assert (nb, ns) == (want["bins"], want["segments"])
    if kind == "halves":
        assert nb >= n - n // 2   # every long document opened its own bin
    assert np.array_equal(got["doc_start"], want["doc_start"])
    assert torch.equal(got["position_ids"][: nb * cap],
                       torch.from_numpy(want["position_ids"]).to(got["position_ids"].device))
    assert np.array_equal(got["cu_seqlens"][: ns + 1], want["cu_seqlens"])


def test_bfd_reproduces_the_packed_workload(qk):
    """The packed workload's position ids are the fullest BFD bin of its drawn
    document lengths, completed by a filler: the device packer's fullest bin
    gives the same ids."""
    w = configs.get("packed")
    lengths = host_bfd.draw_lengths(gen.rng(w.seed, gen.S_DOCS), w.doc_len_min, w.doc_len_max,
                                    pool_tokens=8 * w.tokens).astype(np.int32)
    say("case bfd packed workload", len(lengths))
    got = device_pack(qk, lengths, w.tokens, 64)
    assert int(got["status"][0]) == 0
    nb = int(got["counts"][0])
    fill = np.zeros(nb, np.int64)
    for i, s in enumerate(got["doc_start"]):
        fill[s // w.tokens] += lengths[i]
    b = int(np.argmax(fill))
    pos = got["position_ids"][b * w.tokens: (b + 1) * w.tokens]
    assert np.array_equal(pos, gen.positions(w))


def _pack_with_guards(qk, L, cap, max_bins):
    """Pack into outputs followed by 64 guard words each; returns the call's
    return code, the status, the counts and whether every guard is intact."""
    n = len(L)
    lt = torch.tensor(np.asarray(L, np.int32), dtype=torch.int32, device="cuda")
    guard = -12345
    pos = torch.full((max_bins * cap + 64,), guard, dtype=torch.int32, device="cuda")
    cu = torch.full((n + max_bins + 1 + 64,), guard, dtype=torch.int32, device="cuda")
    ds = torch.full((n + 64,), guard, dtype=torch.int32, device="cuda")
    counts = torch.full((2 + 64,), guard, dtype=torch.int32, device="cuda")
    status = torch.full((1 + 64,), guard, dtype=torch.int32, device="cuda")
    ws = torch.empty(qk.lib.qknr_bfd_workspace_bytes(n, max_bins), dtype=torch.uint8,
                     device="cuda")
    st = qk.lib.qknr_bfd_pack(lt.data_ptr(), n, cap, max_bins, ds.data_ptr(), pos.data_ptr(),
                              cu.data_ptr(), counts.data_ptr(), status.data_ptr(),
                              ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    intact = all(bool(torch.all(t[n_used:] == guard))
                 for t, n_used in ((pos, max_bins * cap), (cu, n + max_bins + 1), (ds, n),
                                   (counts, 2), (status, 1)))
    return st, int(status[0]), counts[:2].tolist(), pos, intact


def test_bfd_status_and_bounds(qk):
    """Too many bins -> status 1, a bad length -> status 2; counts {0, 0}, and
    nothing is written beyond the outputs' extents (guard words intact)."""
    say("case bfd status")
    cap, max_bins = 10, 3
    for L, want in (([7, 7, 7, 7], 1), ([3, 0, 4], 2), ([3, 11, 4], 2), ([5, 5, 5, 5, 5, 5], 0)):
        st, status, counts, pos, intact = _pack_with_guards(qk, L, cap, max_bins)
        assert st == 0
        assert status == want
        assert intact
        if want:
            assert counts == [0, 0]
        else:
            o = oracle.bfd_pack(np.array(L, np.int32), cap, max_bins)
            assert counts == [o["bins"], o["segments"]]
            assert pos[: o["bins"] * cap].cpu().numpy().tolist() == o["position_ids"].tolist()


@pytest.mark.parametrize("cap,max_bins", [(1000, 100), (1000, 1500), (500, 3000), (1 << 20, 70)])
def test_bfd_too_many_bins_on_every_placement(qk, cap, max_bins):
    """One document more than max_bins opens bins: status 1 with counts {0, 0}
    and the guards intact, on the workgroup placements (1, 2 and 4 bins per
    thread) and on the capacity-2^20 loop; a bad length gives status 2 there
    too, and max_bins documents fit (status 0, as the oracle)."""
    say("case bfd overflow", cap, max_bins)
    g = np.random.default_rng(max_bins)
    over = g.permutation(np.concatenate([np.full(max_bins + 1, cap // 2 + 1),
                                         g.integers(1, cap // 2, size=max_bins // 2)]))
    st, status, counts, _, intact = _pack_with_guards(qk, over, cap, max_bins)
    assert (st, status, counts, intact) == (0, 1, [0, 0], True)
    assert oracle.bfd_pack(over.astype(np.int32), cap, max_bins)["status"] == 1
    bad = np.concatenate([over[:10], [cap + 1]])
    st, status, counts, _, intact = _pack_with_guards(qk, bad, cap, max_bins)
    assert (st, status, counts, intact) == (0, 2, [0, 0], True)
    fits = np.full(max_bins, cap // 2 + 1)
    st, status, counts, pos, intact = _pack_with_guards(qk, fits, cap, max_bins)
    o = oracle.bfd_pack(fits.astype(np.int32), cap, max_bins)
    # every bin: the document, then a filler segment for the rest
    assert (o["status"], o["bins"], o["segments"]) == (0, max_bins, 2 * max_bins)
    assert (st, status, counts, intact) == (0, 0, [max_bins, 2 * max_bins], True)
    assert torch.equal(pos[: max_bins * cap], torch.from_numpy(o["position_ids"]).cuda())


def test_bfd_then_qknr_on_the_packed_buffer(qk):
    """The packer's position ids feed the forward directly: documents packed on
    the device and rotated equal each document rotated alone (positions
    0..L-1), bit for bit."""
    g = np.random.default_rng(11)
    cap, H, D = 512, 4, 64
    L = np.clip(np.rint(np.exp(g.uniform(np.log(8), np.log(cap), 40))), 1, cap).astype(np.int32)
    say("case bfd -> qknr")
    r = qk.qknr_bfd_pack(torch.from_numpy(L).cuda(), cap, 40)
    torch.cuda.synchronize()
    nb = int(r["counts"][0])
    T = nb * cap
    pos = r["position_ids"][:T].contiguous()
    q = torch.randn(T, H, D, device="cuda").to(torch.bfloat16)
    k = torch.randn(T, 1, D, device="cuda").to(torch.bfloat16)
    w = torch.ones(D, dtype=torch.bfloat16, device="cuda")
    yq, _ = qk.qknr_fwd(q, k, w, w, pos, D, 1e-6, 1e4)
    starts = r["doc_start"].cpu().numpy()
    for i in range(0, len(L), 7):
        s, n = int(starts[i]), int(L[i])
        alone, _ = qk.qknr_fwd(q[s: s + n].contiguous(), k[s: s + n].contiguous(), w, w,
                               torch.arange(n, dtype=torch.int32, device="cuda"), D, 1e-6, 1e4)
        assert torch.equal(alone, yq[s: s + n])

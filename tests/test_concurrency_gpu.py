"""The library is re-entrant per stream: host threads calling every entry point
at once, each on its own stream with its own outputs and workspaces, give
results bit-identical to the same calls made one after another.  (The
library's per-device caches of resident workgroup counts are filled while
the threads race.)
"""

import threading

import numpy as np
import pytest
import torch

from helpers import to_device
from workloads import gen

pytestmark = pytest.mark.gpu

HW = 16


@pytest.fixture(scope="module")
def qk():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import qk_norm_rope_amd
    torch.cuda.set_device(0)
    return qk_norm_rope_amd


def job(qk, case, stream):
    """One thread's work: dense, options, norm groups and the packer."""
    q, k, wq, wk, hwq, hwk, bq, bk, pos, dyq, dyk, lengths = case
    out = []
    with torch.cuda.stream(stream):
        for _ in range(3):
            yq, yk = qk.qknr_fwd(q, k, wq, wk, pos, 64, 1e-6, 1e6)
            out += [yq, yk]
            out += list(qk.qknr_bwd(q, k, wq, wk, pos, dyq, dyk, 64, 1e-6, 1e6))
            out += list(qk.qknr_fwd_opt(q, k, wq, wk, pos, 64, 1e-6, 1e6, flags=8, bq=bq[0],
                                        bk=bk[0], inv_freq=[1e6 ** (-i / 32) for i in range(32)]))
            out += list(qk.qknr_fwd_opt(q, k, hwq, hwk, pos, 64, 1e-6, 1e6, flags=HW, bq=bq,
                                        bk=bk, norm_groups=(q.shape[1] // k.shape[1], k.shape[1])))
            out += [t for t in qk.qknr_bwd_opt(q, k, hwq, hwk, pos, dyq, dyk, 64, 1e-6, 1e6,
                                               flags=HW, bias_grads=True,
                                               norm_groups=(q.shape[1] // k.shape[1],
                                                            k.shape[1])) if t is not None]
            r = qk.qknr_bfd_pack(lengths, 4096, 256)
            out += [r["doc_start"], r["counts"]]
    stream.synchronize()
    return out


def make_case(seed, T, hq, hkv):
    D, dt = 64, "bf16"
    inp = gen.random_case(seed=seed, tokens=T, hq=hq, hkv=hkv, head_dim=D, dtype=dt, scale=1.0,
                          max_pos=50000, backward=True)
    g = np.random.default_rng(seed)
    dev = {key: to_device(val, dt) for key, val in inp.items() if key != "pos"}
    hwq = to_device(gen.encode(1 + 0.1 * g.standard_normal((hq, D)), dt), dt)
    hwk = to_device(gen.encode(1 + 0.1 * g.standard_normal((hkv, D)), dt), dt)
    bq = to_device(gen.encode(0.1 * g.standard_normal((hq, D)), dt), dt)
    bk = to_device(gen.encode(0.1 * g.standard_normal((hkv, D)), dt), dt)
    lengths = torch.from_numpy(g.integers(1, 4097, size=300).astype(np.int32)).cuda()
    return (dev["q"], dev["k"], dev["wq"], dev["wk"], hwq, hwk, bq, bk,
            torch.from_numpy(inp["pos"]).cuda(), dev["dyq"], dev["dyk"], lengths)


def test_threads_on_their_own_streams(qk):
    cases = [make_case(40 + i, 2048 + 97 * i, 14, 2) for i in range(4)]
    torch.cuda.synchronize()
    seq = [job(qk, c, torch.cuda.Stream()) for c in cases]
    results = [None] * len(cases)
    errors = []

    def run(i):
        try:
            results[i] = job(qk, cases[i], torch.cuda.Stream())
        except Exception as e:  # pragma: no cover - reported below
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(cases))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for a, b in zip(seq, results):
        assert len(a) == len(b)
        for x, y in zip(a, b):
            assert torch.equal(x, y)

"""qknr_bwd_noalloc (the backward whose weight-gradient partials live in the
library's static device array) against qknr_bwd with a workspace, through the C
ABI: two calls in a row, the second with a smaller input (the array keeps the
first call's partials), each bit-identical to qknr_bwd and within the parity
rules of the oracle."""

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


@pytest.fixture(scope="module")
def qk():
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    import qk_norm_rope_amd
    torch.cuda.set_device(0)
    return qk_norm_rope_amd


def _case(qk, inp, dtype, R, eps, theta, what):
    print("case", what, flush=True)
    d = {key: (torch.from_numpy(np.ascontiguousarray(v)).cuda() if key == "pos"
               else to_device(v, dtype)) for key, v in inp.items()}
    args = (R, eps, theta)
    ref = qk.qknr_bwd(d["q"], d["k"], d["wq"], d["wk"], d["pos"], d["dyq"], d["dyk"], *args)
    out = [torch.full_like(d["q"], 7.0), torch.full_like(d["k"], 7.0),
           torch.full_like(d["wq"], 7.0), torch.full_like(d["wk"], 7.0)]
    got = qk.qknr_bwd_noalloc(d["q"], d["k"], d["wq"], d["wk"], d["pos"], d["dyq"], d["dyk"],
                              *args, *out)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dwq", "dwk"), got, ref):
        assert torch.equal(a.view(torch.int16) if dtype == "bf16" else a.view(torch.int32),
                           b.view(torch.int16) if dtype == "bf16" else b.view(torch.int32)), name
    dec = lambda a: oracle.decode(a, dtype)  # noqa: E731
    o = oracle.bwd(dec(inp["q"]), dec(inp["k"]), dec(inp["wq"]), dec(inp["wk"]), inp["pos"],
                   dec(inp["dyq"]), dec(inp["dyk"]), *args, threads=THREADS)
    for name, a, ov in zip(("dq", "dk", "dwq", "dwk"), got, o):
        compare(gpu_values(a, dtype), ov, dtype, "%s:%s" % (what, name),
                row_sum=name.startswith("dw"))


def test_no_alloc_backward_equals_workspace_backward(qk):
    # first call: 8192 tokens of the Qwen2.5-0.5B-shaped workload (the most
    # partial rows the backward uses, 512)
    w = configs.QWEN05
    inp = gen.make_inputs(w, 0, 8192, backward=True)
    _case(qk, inp, w.dtype, w.rotary_dim, w.eps, w.theta, "no-alloc qwen05[0:8192]")
    # second call, smaller: fewer partial rows than the array still holds
    inp = gen.random_case(seed=21, tokens=301, hq=8, hkv=2, head_dim=128, dtype="bf16",
                          scale=1.5, max_pos=100000)
    _case(qk, inp, "bf16", 64, 1e-5, 1e4, "no-alloc 301 tokens D=128 R=64")
    # and fp32, smaller again
    inp = gen.random_case(seed=22, tokens=37, hq=3, hkv=1, head_dim=64, dtype="f32",
                          scale=1.0, max_pos=4096)
    _case(qk, inp, "f32", 64, 1e-6, 1e4, "no-alloc 37 tokens fp32")


def test_no_alloc_zero_tokens_and_errors(qk):
    z = torch.empty((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    zk = torch.empty((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    pos = torch.empty(0, dtype=torch.int32, device="cuda")
    qk.qknr_bwd_noalloc(z, zk, w, w, pos, z, zk, 64, 1e-6, 1e4, z, zk, w.clone(), w.clone())
    q = torch.zeros((4, 2, 64), dtype=torch.bfloat16, device="cuda")
    p4 = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(qk.QknrError) as e:
        qk.qknr_bwd_noalloc(q, q, w, w, p4, q, q, 24, 1e-6, 1e4, q.clone(), q.clone(), w.clone(),
                            w.clone())
    assert e.value.status == 2
    torch.cuda.synchronize()

"""Seeded synthetic inputs for the QK-Norm + RoPE workloads.

This module serves both the HIP path and the oracle and therefore holds none
of the method's arithmetic: only random draws, the storage encoding of the
drawn values (fp64 -> fp32 -> bf16, round-to-nearest-even at each step) and the
position ids.

Every tensor is drawn in chunks of ``CHUNK`` tokens, and chunk ``c`` of stream
``s`` comes from ``numpy.random.default_rng([seed, s, c])`` (PCG64 seeded by a
SeedSequence).  Any token range can therefore be regenerated on its own, which
lets a test draw only the tokens it samples from a full-size workload.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import bfd
from .configs import Workload

CHUNK = 1024

S_Q, S_K, S_DYQ, S_DYK, S_WQ, S_WK, S_OUT_Q, S_OUT_K, S_DOCS = range(1, 10)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def rng(seed: int, stream: int, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, stream, chunk])


def f64_to_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, np.float64).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the uint16 bits.
    Inputs here are finite and far from the overflow threshold."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


def encode(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Storage encoding: fp64 -> fp32 (RNE) and, for bf16, fp32 -> bf16 (RNE)."""
    x32 = f64_to_f32(x64)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def storage_dtype(dtype: str):
    return np.uint16 if dtype == "bf16" else np.float32


def positions(w: Workload) -> np.ndarray:
    """int32 [tokens]: 0..seq-1 per sequence, or per packed document."""
    if w.packed:
        return packed_layout(w)[0]
    t = np.arange(w.tokens, dtype=np.int64)
    return (t % w.seq).astype(np.int32)


def packed_layout(w: Workload):
    """(position_ids, cu_seqlens) of the packed buffer of a packed workload."""
    lengths = bfd.draw_lengths(rng(w.seed, S_DOCS), w.doc_len_min, w.doc_len_max,
                               pool_tokens=8 * w.tokens)
    docs = bfd.pack_one_buffer(lengths, w.tokens)
    pos = np.concatenate([np.arange(L, dtype=np.int32) for L in docs])
    cu = np.concatenate([[0], np.cumsum(docs)]).astype(np.int64)
    assert pos.shape[0] == w.tokens
    return pos, cu


def weights(w: Workload):
    """Norm weights 1 + 0.1*N(0,1), one [D] vector for Q and one for K."""
    wq = 1.0 + 0.1 * rng(w.seed, S_WQ).standard_normal(w.head_dim)
    wk = 1.0 + 0.1 * rng(w.seed, S_WK).standard_normal(w.head_dim)
    return encode(wq, w.dtype), encode(wk, w.dtype)


def outlier_channels(w: Workload, which: str) -> np.ndarray:
    """Flattened [H*D] channel indices scaled by ``outlier_gain``: round(frac*H*D)
    of them, drawn without replacement, fixed across tokens."""
    if w.outlier_frac <= 0:
        return np.zeros(0, np.int64)
    h = w.hq if which == "q" else w.hkv
    n = int(round(w.outlier_frac * h * w.head_dim))
    g = rng(w.seed, S_OUT_Q if which == "q" else S_OUT_K)
    return np.sort(g.choice(h * w.head_dim, size=n, replace=False))


_STREAM = {"q": S_Q, "k": S_K, "dyq": S_DYQ, "dyk": S_DYK}


def _heads(w: Workload, which: str) -> int:
    return w.hq if which in ("q", "dyq") else w.hkv


def _chunk_values(w: Workload, which: str, c: int, t0: int, t1: int, out: np.ndarray,
                  outl: np.ndarray):
    """Fill ``out`` ([t1-t0, H, D], storage dtype) with chunk c's values."""
    h = _heads(w, which)
    width = h * w.head_dim
    x = rng(w.seed, _STREAM[which], c).standard_normal((t1 - t0, width))
    if which in ("q", "k"):
        if w.value_scale != 1.0:
            x *= w.value_scale
        if outl.size:
            x[:, outl] *= w.outlier_gain
    out[...] = encode(x, w.dtype).reshape(t1 - t0, h, w.head_dim)


def tensor(w: Workload, which: str, t0: int = 0, t1: int | None = None,
           threads: int | None = None) -> np.ndarray:
    """Stored values of ``which`` in {"q", "k", "dyq", "dyk"} for tokens [t0, t1).
    Returns [t1-t0, H, D] in the storage dtype (uint16 bits for bf16)."""
    t1 = w.tokens if t1 is None else t1
    assert 0 <= t0 <= t1 <= w.tokens
    h = _heads(w, which)
    out = np.empty((t1 - t0, h, w.head_dim), storage_dtype(w.dtype))
    outl = outlier_channels(w, which) if which in ("q", "k") else np.zeros(0, np.int64)
    jobs = []
    for c in range(t0 // CHUNK, -(-t1 // CHUNK) if t1 > 0 else 0):
        a, b = c * CHUNK, min((c + 1) * CHUNK, w.tokens)
        lo, hi = max(a, t0), min(b, t1)
        if lo >= hi:
            continue
        jobs.append((c, a, b, lo, hi))

    def run(job):
        c, a, b, lo, hi = job
        if lo == a and hi == b:
            _chunk_values(w, which, c, a, b, out[a - t0:b - t0], outl)
        else:
            tmp = np.empty((b - a, h, w.head_dim), out.dtype)
            _chunk_values(w, which, c, a, b, tmp, outl)
            out[lo - t0:hi - t0] = tmp[lo - a:hi - a]

    n = threads if threads is not None else _threads()
    if n <= 1 or len(jobs) <= 1:
        for j in jobs:
            run(j)
    else:
        with ThreadPoolExecutor(min(n, len(jobs))) as ex:
            list(ex.map(run, jobs))
    return out


def tokens_sample(w: Workload, which: str, idx: np.ndarray) -> np.ndarray:
    """Stored values of ``which`` at the given token indices (any order)."""
    idx = np.asarray(idx, np.int64)
    h = _heads(w, which)
    out = np.empty((idx.size, h, w.head_dim), storage_dtype(w.dtype))
    chunks = np.unique(idx // CHUNK)
    for c in chunks:
        a = int(c) * CHUNK
        b = min(a + CHUNK, w.tokens)
        block = tensor(w, which, a, b, threads=1)
        sel = np.nonzero(idx // CHUNK == c)[0]
        out[sel] = block[idx[sel] - a]
    return out


def make_inputs(w: Workload, t0: int = 0, t1: int | None = None, backward: bool | None = None,
                threads: int | None = None) -> dict:
    """All inputs of a workload for tokens [t0, t1): q, k, wq, wk, pos and, when
    the backward is included, the upstream gradients dyq, dyk."""
    t1 = w.tokens if t1 is None else t1
    backward = w.backward if backward is None else backward
    wq, wk = weights(w)
    d = {
        "q": tensor(w, "q", t0, t1, threads),
        "k": tensor(w, "k", t0, t1, threads),
        "wq": wq,
        "wk": wk,
        "pos": positions(w)[t0:t1].copy(),
    }
    if backward:
        d["dyq"] = tensor(w, "dyq", t0, t1, threads)
        d["dyk"] = tensor(w, "dyk", t0, t1, threads)
    return d


def random_case(seed: int, tokens: int, hq: int, hkv: int, head_dim: int, dtype: str,
                scale: float = 1.0, max_pos: int = 4096, backward: bool = True) -> dict:
    """Small free-form case for sweeps: random positions in [0, max_pos)."""
    g = np.random.default_rng([seed, 0xC0FFEE, tokens, hq, hkv, head_dim])
    d = {
        "q": encode(scale * g.standard_normal((tokens, hq, head_dim)), dtype),
        "k": encode(scale * g.standard_normal((tokens, hkv, head_dim)), dtype),
        "wq": encode(1.0 + 0.1 * g.standard_normal(head_dim), dtype),
        "wk": encode(1.0 + 0.1 * g.standard_normal(head_dim), dtype),
        "pos": g.integers(0, max_pos, size=tokens).astype(np.int32),
    }
    if backward:
        d["dyq"] = encode(g.standard_normal((tokens, hq, head_dim)), dtype)
        d["dyk"] = encode(g.standard_normal((tokens, hkv, head_dim)), dtype)
    return d

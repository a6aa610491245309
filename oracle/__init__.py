"""fp64 CPU oracle for per-head QK-Norm followed by RoPE (test infrastructure).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path (``qk_norm_rope_amd``)
never imports this package, and this package imports nothing from it.

The arithmetic lives in ``qknr_oracle.c`` (plain C, fp64 scalar loops, built
with ``-O2 -ffp-contract=off``); this module only marshals NumPy arrays into it
and splits token ranges over host threads.  The definitions it follows are
listed in the C file's header: RMSNorm as static weight times a per-row
inverse-RMS scalar (abstract of "QK-Normed MLA: QK normalization without full
key caching"), applied per head (QG-MIL and HobbyLM abstracts), then RoPE on
the first ``rotary_dim`` channels (abstract of "Fractional Rotation, Full
Potential? Investigating Performance and Convergence of Partial RoPE").

Input decoding: bf16 inputs arrive as their uint16 bit patterns; a bf16 value
is the fp32 whose top 16 bits are those bits, so widening is exact.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qknr_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test that plants mistakes in a copy of the C source points this at the
# mutant's build; nothing else sets it.
_LIB_OVERRIDE = os.environ.get("QKNR_ORACLE_LIB")
_lock = threading.Lock()
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_u16p = ctypes.POINTER(ctypes.c_uint16)


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/liboracle.so``."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
        lib.oracle_fwd.restype = ctypes.c_int
        lib.oracle_fwd.argtypes = [_dp, _dp, _dp, _dp, _ip, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                   ctypes.c_double, _dp, _dp]
        lib.oracle_bwd.restype = ctypes.c_int
        lib.oracle_bwd.argtypes = [_dp, _dp, _dp, _dp, _ip, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                   ctypes.c_double, _dp, _dp, _dp, _dp, _dp, _dp]
        lib.oracle_fwd_ex.restype = ctypes.c_int
        lib.oracle_fwd_ex.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _ip, ctypes.c_int64,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_double, ctypes.c_double, ctypes.c_int, _dp,
                                      ctypes.c_double, _dp, _dp]
        lib.oracle_bwd_ex.restype = ctypes.c_int
        lib.oracle_bwd_ex.argtypes = [_dp, _dp, _dp, _dp, _ip, ctypes.c_int64, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                      ctypes.c_double, ctypes.c_int, _dp, ctypes.c_double, _dp,
                                      _dp, _dp, _dp, _dp, _dp, _dp, _dp]
        lib.oracle_fwd_gen.restype = ctypes.c_int
        lib.oracle_fwd_gen.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _ip, ctypes.c_int64,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_double, ctypes.c_double, ctypes.c_int, _dp,
                                       ctypes.c_double, ctypes.c_int, ctypes.c_int, _dp, _dp]
        lib.oracle_bwd_gen.restype = ctypes.c_int
        lib.oracle_bwd_gen.argtypes = [_dp, _dp, _dp, _dp, _ip, ctypes.c_int64, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                       ctypes.c_double, ctypes.c_int, _dp, ctypes.c_double,
                                       ctypes.c_int, ctypes.c_int, _dp, _dp, _dp, _dp, _dp, _dp,
                                       _dp, _dp]
        lib.oracle_bfd_pack.restype = ctypes.c_int
        lib.oracle_bfd_pack.argtypes = [_ip, ctypes.c_int, ctypes.c_int, ctypes.c_int, _ip, _ip, _ip,
                                        _ip]
        lib.oracle_rope_cos_sin.restype = None
        lib.oracle_rope_cos_sin.argtypes = [ctypes.c_int64, ctypes.c_double, ctypes.c_int, _dp, _dp]
        lib.oracle_rope_cos_sin_ex.restype = None
        lib.oracle_rope_cos_sin_ex.argtypes = [ctypes.c_int64, ctypes.c_double, ctypes.c_int,
                                               ctypes.c_int, _dp, _dp]
        lib.oracle_rope_cos_sin_gen.restype = None
        lib.oracle_rope_cos_sin_gen.argtypes = [ctypes.c_int64, ctypes.c_double, ctypes.c_int,
                                                ctypes.c_int, _dp, ctypes.c_double, _dp, _dp]
        lib.oracle_round_bf16.restype = None
        lib.oracle_round_bf16.argtypes = [_dp, ctypes.c_int64, _u16p]
        _lib = lib
        return lib


def _ptr(a, t):
    return a.ctypes.data_as(t)


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored inputs to fp64 exactly.  ``dtype`` is "bf16" (uint16 bit
    patterns) or "f32"."""
    if dtype == "bf16":
        a = np.ascontiguousarray(a, dtype=np.uint16)
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError("dtype must be 'bf16' or 'f32'")


def eps_as_used(eps: float) -> float:
    """eps is handed to the kernels as fp32; the oracle adds the same value."""
    return float(np.float32(eps))


# Convention flags (the C file's ORACLE_* values).
INTERLEAVED = 1      # rotate pairs (2i, 2i+1) instead of (i, i + R/2)
FREQ_HEAD_DIM = 2    # theta_i = theta^(-2i/D) instead of theta^(-2i/R)
LAYERNORM = 4        # subtract the row mean before scaling (QK-LayerNorm)
HEAD_WEIGHTS = 8     # weights, biases and their gradients are [H, D] (one vector per head)


def flags_of(interleaved: bool = False, freq_head_dim: bool = False, layernorm: bool = False,
             head_weights: bool = False) -> int:
    return ((INTERLEAVED if interleaved else 0) | (FREQ_HEAD_DIM if freq_head_dim else 0)
            | (LAYERNORM if layernorm else 0) | (HEAD_WEIGHTS if head_weights else 0))


def _opt(a, n=None):
    """None, or a contiguous fp64 array (of length n when given)."""
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.float64)
    if n is not None:
        assert a.shape == (n,), (a.shape, n)
    return a


def _optp(a):
    return None if a is None else _ptr(a, _dp)


def rope_cos_sin(pos: int, theta: float, rotary_dim: int, freq_denom: int | None = None,
                 inv_freq=None, attention_factor: float = 1.0):
    """fp32-rounded a*cos/a*sin of pos*theta_i, i < R/2, as fp64 arrays, with
    theta_i = theta^(-2i/denom) (denom = rotary_dim unless given) or the
    table inv_freq, and a = attention_factor."""
    lib = _load()
    h = rotary_dim // 2
    c = np.zeros(max(h, 1), np.float64)
    s = np.zeros(max(h, 1), np.float64)
    if inv_freq is not None or attention_factor != 1.0:
        tab = _opt(inv_freq, h)
        lib.oracle_rope_cos_sin_gen(int(pos), float(theta), int(rotary_dim),
                                    int(freq_denom or rotary_dim), _optp(tab),
                                    float(attention_factor), _ptr(c, _dp), _ptr(s, _dp))
    elif freq_denom is None:
        lib.oracle_rope_cos_sin(int(pos), float(theta), int(rotary_dim), _ptr(c, _dp), _ptr(s, _dp))
    else:
        lib.oracle_rope_cos_sin_ex(int(pos), float(theta), int(rotary_dim), int(freq_denom),
                                   _ptr(c, _dp), _ptr(s, _dp))
    return c[:h], s[:h]


def round_bf16(v: np.ndarray) -> np.ndarray:
    """One-step round-to-nearest-even of fp64 values to bf16; returns uint16 bits."""
    lib = _load()
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    lib.oracle_round_bf16(_ptr(v, _dp), v.size, _ptr(out, _u16p))
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return decode(bits, "bf16")


def _ranges(tokens: int, threads: int):
    threads = max(1, min(threads, tokens)) if tokens > 0 else 1
    step = -(-tokens // threads) if tokens > 0 else 0
    return [(a, min(tokens, a + step)) for a in range(0, tokens, step)] if tokens > 0 else []


def _as_f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _wshape(flags, H, D):
    return (H, D) if flags & HEAD_WEIGHTS else (D,)


def fwd(q, k, wq, wk, pos, rotary_dim: int, eps: float, theta: float, threads: int = 1,
        flags: int = 0, bq=None, bk=None, inv_freq=None, attention_factor: float = 1.0,
        norm_groups=None):
    """Forward.  q: [T, Hq, D], k: [T, Hkv, D], wq/wk: [D] (fp64 values; [Hq, D] /
    [Hkv, D] with HEAD_WEIGHTS), pos: [T] int, flags: INTERLEAVED |
    FREQ_HEAD_DIM | LAYERNORM | HEAD_WEIGHTS; optional biases bq/bk (shaped like
    the weights), frequency table inv_freq [R/2], attention factor, and
    norm_groups = (gq, gk), the heads of q and of k that share one inverse RMS
    (None: per head, through the per-row path).  Returns fp64 (yq, yk) of the
    shapes of q and k."""
    lib = _load()
    q, k = _as_f64(q), _as_f64(k)
    T, hq, D = q.shape
    hkv = k.shape[1]
    wq, wk = _as_f64(wq), _as_f64(wk)
    assert wq.shape == _wshape(flags, hq, D) and wk.shape == _wshape(flags, hkv, D)
    bq = None if bq is None else _as_f64(bq)
    bk = None if bk is None else _as_f64(bk)
    assert bq is None or bq.shape == wq.shape
    assert bk is None or bk.shape == wk.shape
    tab = _opt(inv_freq, rotary_dim // 2)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    assert k.shape == (T, hkv, D) and pos.shape == (T,)
    gen = norm_groups is not None or bool(flags & HEAD_WEIGHTS)
    gq, gk = norm_groups if norm_groups is not None else (1, 1)
    yq = np.empty_like(q)
    yk = np.empty_like(k)
    e = eps_as_used(eps)

    def run(rng):
        a, b = rng
        common = (_ptr(q[a:b], _dp), _ptr(k[a:b], _dp), _ptr(wq, _dp), _ptr(wk, _dp), _optp(bq),
                  _optp(bk), _ptr(pos[a:b], _ip), b - a, hq, hkv, D, int(rotary_dim), e,
                  float(theta), int(flags), _optp(tab), float(attention_factor))
        if gen:
            rc = lib.oracle_fwd_gen(*common, int(gq), int(gk), _ptr(yq[a:b], _dp),
                                    _ptr(yk[a:b], _dp))
        else:
            rc = lib.oracle_fwd_ex(*common, _ptr(yq[a:b], _dp), _ptr(yk[a:b], _dp))
        if rc != 0:
            raise ValueError("oracle_fwd rejected the sizes")

    rs = _ranges(T, threads)
    if len(rs) <= 1:
        for r in rs:
            run(r)
    else:
        with ThreadPoolExecutor(len(rs)) as ex:
            list(ex.map(run, rs))
    return yq, yk


def bwd(q, k, wq, wk, pos, dyq, dyk, rotary_dim: int, eps: float, theta: float,
        threads: int = 1, flags: int = 0, inv_freq=None, attention_factor: float = 1.0,
        bias_grads: bool = False, norm_groups=None):
    """Backward.  Returns fp64 (dq, dk, dwq, dwk), and dbq, dbk after them with
    bias_grads; weight and bias gradients have the weights' shapes.  dw (db)
    is the sum over every row of its tensor; with several threads each token
    range is summed on its own and the range sums are added in range order.
    norm_groups as in fwd."""
    lib = _load()
    tab = _opt(inv_freq, rotary_dim // 2)
    q, k, wq, wk = _as_f64(q), _as_f64(k), _as_f64(wq), _as_f64(wk)
    dyq, dyk = _as_f64(dyq), _as_f64(dyk)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    T, hq, D = q.shape
    hkv = k.shape[1]
    assert dyq.shape == q.shape and dyk.shape == k.shape
    assert wq.shape == _wshape(flags, hq, D) and wk.shape == _wshape(flags, hkv, D)
    gen = norm_groups is not None or bool(flags & HEAD_WEIGHTS)
    gq, gk = norm_groups if norm_groups is not None else (1, 1)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    e = eps_as_used(eps)
    rs = _ranges(T, threads)
    parts = [(np.zeros(wq.shape), np.zeros(wk.shape), np.zeros(wq.shape), np.zeros(wk.shape))
             for _ in rs]

    def run(i):
        a, b = rs[i]
        dwq_i, dwk_i, dbq_i, dbk_i = parts[i]
        head = (_ptr(q[a:b], _dp), _ptr(k[a:b], _dp), _ptr(wq, _dp), _ptr(wk, _dp),
                _ptr(pos[a:b], _ip), b - a, hq, hkv, D, int(rotary_dim), e, float(theta),
                int(flags), _optp(tab), float(attention_factor))
        tail = (_ptr(dyq[a:b], _dp), _ptr(dyk[a:b], _dp), _ptr(dq[a:b], _dp), _ptr(dk[a:b], _dp),
                _ptr(dwq_i, _dp), _ptr(dwk_i, _dp),
                _ptr(dbq_i, _dp) if bias_grads else None,
                _ptr(dbk_i, _dp) if bias_grads else None)
        if gen:
            rc = lib.oracle_bwd_gen(*head, int(gq), int(gk), *tail)
        else:
            rc = lib.oracle_bwd_ex(*head, *tail)
        if rc != 0:
            raise ValueError("oracle_bwd rejected the sizes")

    if len(rs) <= 1:
        for i in range(len(rs)):
            run(i)
    else:
        with ThreadPoolExecutor(len(rs)) as ex:
            list(ex.map(run, range(len(rs))))
    sums = [np.zeros(a.shape) for a in parts[0]] if parts else [np.zeros(wq.shape), np.zeros(wk.shape),
                                                                 np.zeros(wq.shape), np.zeros(wk.shape)]
    for part in parts:
        for acc, v in zip(sums, part):
            acc += v
    dwq, dwk, dbq, dbk = sums
    if bias_grads:
        return dq, dk, dwq, dwk, dbq, dbk
    return dq, dk, dwq, dwk


def bfd_pack(lengths, capacity: int, max_bins: int):
    """Best-Fit-Decreasing packing of documents into buffers of `capacity`
    tokens (tie-breaks in the C oracle's header).  Returns a dict: status (0
    ok, 1 more than max_bins bins, 2 a length outside [1, capacity]), and when
    0: doc_start [n] (first token of each document), position_ids [bins *
    capacity], cu_seqlens [segments + 1], bins, segments."""
    lib = _load()
    L = np.ascontiguousarray(lengths, dtype=np.int32)
    n = int(L.shape[0])
    doc_start = np.full(max(n, 1), -1, np.int32)
    pos = np.full(max(1, max_bins * capacity), -1, np.int32)
    cu = np.full(n + max_bins + 1, -1, np.int32)
    counts = np.zeros(2, np.int32)
    st = lib.oracle_bfd_pack(_ptr(L, _ip) if n else None, n, int(capacity), int(max_bins),
                             _ptr(doc_start, _ip), _ptr(pos, _ip), _ptr(cu, _ip), _ptr(counts, _ip))
    out = {"status": int(st)}
    if st == 0:
        nb, ns = int(counts[0]), int(counts[1])
        out.update(doc_start=doc_start[:n].copy(), position_ids=pos[: nb * capacity].copy(),
                   cu_seqlens=cu[: ns + 1].copy(), bins=nb, segments=ns)
    return out

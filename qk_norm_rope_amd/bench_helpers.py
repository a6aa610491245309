"""ctypes binding of libqknr_bench.so: plain streaming kernels that measure the
achievable HBM bandwidth, an empty kernel that measures a dispatch, and a fill
that evicts caches (declared in include/qknr_bench.h).
Used by the benchmark; not part of the operation."""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG, "libqknr_bench.so")


def _load():
    if not os.path.exists(lib_path):
        raise ImportError("libqknr_bench.so is not built (expected at %s); run "
                          "`python -m qk_norm_rope_amd.build`" % lib_path)
    L = ctypes.CDLL(lib_path)
    V, sz = ctypes.c_void_p, ctypes.c_size_t
    L.qknr_bench_copy.restype = ctypes.c_int
    L.qknr_bench_copy.argtypes = [V, V, sz, V]
    L.qknr_bench_stream2.restype = ctypes.c_int
    L.qknr_bench_stream2.argtypes = [V, V, V, sz, V]
    L.qknr_bench_flush.restype = ctypes.c_int
    L.qknr_bench_flush.argtypes = [V, sz, ctypes.c_uint32, V]
    L.qknr_bench_empty.restype = ctypes.c_int
    L.qknr_bench_empty.argtypes = [V]
    return L


lib = _load()


def _stream(t: torch.Tensor, stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.current_stream(t.device).cuda_stream


def _ok(st: int, where: str):
    if st != 0:
        raise RuntimeError("%s failed with status %d" % (where, st))


def copy(src: torch.Tensor, dst: torch.Tensor, stream=None):
    """Plain streaming copy of src's bytes into dst."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst smaller than src")
    _ok(lib.qknr_bench_copy(src.data_ptr(), dst.data_ptr(), n, _stream(src, stream)), "copy")


def stream2(a: torch.Tensor, b: torch.Tensor, dst: torch.Tensor, stream=None):
    """dst = a ^ b over a's bytes (two reads, one write)."""
    n = a.numel() * a.element_size()
    if b.numel() * b.element_size() < n or dst.numel() * dst.element_size() < n:
        raise ValueError("b or dst smaller than a")
    _ok(lib.qknr_bench_stream2(a.data_ptr(), b.data_ptr(), dst.data_ptr(), n, _stream(a, stream)),
        "stream2")


def flush(buf: torch.Tensor, seed: int = 0, stream=None):
    """Overwrite buf (evicts other data from L2 and the Infinity Cache)."""
    _ok(lib.qknr_bench_flush(buf.data_ptr(), buf.numel() * buf.element_size(),
                             int(seed) & 0xFFFFFFFF, _stream(buf, stream)), "flush")


def empty(stream=None):
    """Launch a kernel that does nothing (the cost of one dispatch)."""
    st = (stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)) \
        if stream is not None else torch.cuda.current_stream().cuda_stream
    _ok(lib.qknr_bench_empty(st), "empty")

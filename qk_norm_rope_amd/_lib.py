"""ctypes binding of libqknr.so (argument marshalling only)."""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG, "libqknr.so")

QKNR_F32 = 0
QKNR_BF16 = 1

_c_void_p = ctypes.c_void_p
_i32, _i64, _f32, _f64, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_size_t


class QknrError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s failed: %s (status %d)" % (where, qknr_status_string(status), status))
        self.status = status


def _load():
    if not os.path.exists(lib_path):
        raise ImportError(
            "libqknr.so is not built (expected at %s); run `python -m qk_norm_rope_amd.build` "
            "or __graft_entry__.build()" % lib_path)
    L = ctypes.CDLL(lib_path)
    L.qknr_fwd.restype = ctypes.c_int
    L.qknr_fwd.argtypes = [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i32,
                           _i32, _i32, _f32, _f64, ctypes.c_int, _c_void_p, _c_void_p, _c_void_p]
    L.qknr_bwd.restype = ctypes.c_int
    L.qknr_bwd.argtypes = [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i32,
                           _i32, _i32, _f32, _f64, ctypes.c_int, _c_void_p, _c_void_p, _c_void_p,
                           _c_void_p, _c_void_p, _c_void_p, _c_void_p, _sz, _c_void_p]
    L.qknr_bwd_workspace_bytes.restype = _sz
    L.qknr_bwd_workspace_bytes.argtypes = [_i64, _i32, _i32, _i32, ctypes.c_int]
    L.qknr_status_string.restype = ctypes.c_char_p
    L.qknr_status_string.argtypes = [ctypes.c_int]
    L.qknr_copy.restype = ctypes.c_int
    L.qknr_copy.argtypes = [_c_void_p, _c_void_p, _sz, _c_void_p]
    L.qknr_flush.restype = ctypes.c_int
    L.qknr_flush.argtypes = [_c_void_p, _sz, ctypes.c_uint32, _c_void_p]
    return L


lib = _load()


def qknr_status_string(status: int) -> str:
    return lib.qknr_status_string(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return QKNR_BF16
    if t.dtype == torch.float32:
        return QKNR_F32
    raise TypeError("q/k must be torch.bfloat16 or torch.float32, got %s" % t.dtype)


def _stream(device, stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.current_stream(device).cuda_stream


def _check(name, t, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _positions(position_ids, tokens, device):
    if position_ids.dtype == torch.int64:
        position_ids = position_ids.to(torch.int32)
    _check("position_ids", position_ids, torch.int32, (tokens,), device)
    return position_ids


def _shapes(q, k):
    if q.dim() != 3 or k.dim() != 3 or q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2]:
        raise ValueError("q must be [tokens, hq, D] and k [tokens, hkv, D]")
    return q.shape[0], q.shape[1], k.shape[1], q.shape[2]


def qknr_fwd(q, k, wq, wk, position_ids, rotary_dim: int, eps: float, theta: float,
             q_out=None, k_out=None, stream=None):
    """RoPE(RMSNorm_wq(q)), RoPE(RMSNorm_wk(k)).  Pass q_out=q / k_out=k for in
    place.  Returns (q_out, k_out)."""
    T, hq, hkv, D = _shapes(q, k)
    dev = q.device
    dt = q.dtype
    for n, t, s in (("q", q, (T, hq, D)), ("k", k, (T, hkv, D)), ("wq", wq, (D,)), ("wk", wk, (D,))):
        _check(n, t, dt, s, dev)
    pos = _positions(position_ids, T, dev)
    q_out = torch.empty_like(q) if q_out is None else q_out
    k_out = torch.empty_like(k) if k_out is None else k_out
    _check("q_out", q_out, dt, (T, hq, D), dev)
    _check("k_out", k_out, dt, (T, hkv, D), dev)
    st = lib.qknr_fwd(q.data_ptr(), k.data_ptr(), wq.data_ptr(), wk.data_ptr(), pos.data_ptr(),
                      T, hq, hkv, D, int(rotary_dim), float(eps), float(theta), _dtype_code(q),
                      q_out.data_ptr(), k_out.data_ptr(), _stream(dev, stream))
    if st != 0:
        raise QknrError(st, "qknr_fwd")
    return q_out, k_out


def qknr_bwd_workspace_bytes(tokens: int, hq: int, hkv: int, head_dim: int, dtype) -> int:
    code = dtype if isinstance(dtype, int) else (QKNR_BF16 if dtype == torch.bfloat16 else QKNR_F32)
    return int(lib.qknr_bwd_workspace_bytes(int(tokens), int(hq), int(hkv), int(head_dim), code))


def qknr_bwd(q, k, wq, wk, position_ids, dq_out, dk_out, rotary_dim: int, eps: float,
             theta: float, dq=None, dk=None, dwq=None, dwk=None, workspace=None, stream=None):
    """Gradients of <dq_out, q_out> + <dk_out, k_out> w.r.t. q, k, wq, wk.
    Returns (dq, dk, dwq, dwk); dwq/dwk are overwritten."""
    T, hq, hkv, D = _shapes(q, k)
    dev = q.device
    dt = q.dtype
    for n, t, s in (("q", q, (T, hq, D)), ("k", k, (T, hkv, D)), ("wq", wq, (D,)), ("wk", wk, (D,)),
                    ("dq_out", dq_out, (T, hq, D)), ("dk_out", dk_out, (T, hkv, D))):
        _check(n, t, dt, s, dev)
    pos = _positions(position_ids, T, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dwq = torch.empty_like(wq) if dwq is None else dwq
    dwk = torch.empty_like(wk) if dwk is None else dwk
    for n, t, s in (("dq", dq, (T, hq, D)), ("dk", dk, (T, hkv, D)), ("dwq", dwq, (D,)), ("dwk", dwk, (D,))):
        _check(n, t, dt, s, dev)
    need = qknr_bwd_workspace_bytes(T, hq, hkv, D, _dtype_code(q))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on %s" % dev)
    wbytes = workspace.numel() * workspace.element_size()
    st = lib.qknr_bwd(q.data_ptr(), k.data_ptr(), wq.data_ptr(), wk.data_ptr(), pos.data_ptr(),
                      T, hq, hkv, D, int(rotary_dim), float(eps), float(theta), _dtype_code(q),
                      dq_out.data_ptr(), dk_out.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                      dwq.data_ptr(), dwk.data_ptr(), workspace.data_ptr(), wbytes,
                      _stream(dev, stream))
    if st != 0:
        raise QknrError(st, "qknr_bwd")
    return dq, dk, dwq, dwk


def qknr_copy(src: torch.Tensor, dst: torch.Tensor, stream=None):
    """Measurement helper: plain streaming copy of src's bytes into dst."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst smaller than src")
    st = lib.qknr_copy(src.data_ptr(), dst.data_ptr(), n, _stream(src.device, stream))
    if st != 0:
        raise QknrError(st, "qknr_copy")


def qknr_flush(buf: torch.Tensor, seed: int = 0, stream=None):
    """Measurement helper: overwrite buf to evict caches."""
    st = lib.qknr_flush(buf.data_ptr(), buf.numel() * buf.element_size(), int(seed) & 0xFFFFFFFF,
                        _stream(buf.device, stream))
    if st != 0:
        raise QknrError(st, "qknr_flush")

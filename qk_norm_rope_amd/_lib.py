"""ctypes binding of libqknr.so (argument marshalling only)."""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG, "libqknr.so")

QKNR_F32 = 0
QKNR_BF16 = 1

QKNR_FLAG_INTERLEAVED = 1     # rotate pairs (2i, 2i+1)
QKNR_FLAG_FREQ_HEAD_DIM = 2   # frequencies theta^(-2i/head_dim)
QKNR_FLAG_NO_WEIGHT = 4       # parameter-free norm (w = 1)
QKNR_FLAG_LAYERNORM = 8       # subtract the row mean first (QK-LayerNorm)
QKNR_FLAG_HEAD_WEIGHTS = 16   # [H, D] weights and biases (one vector per head)

_c_void_p = ctypes.c_void_p
_i32, _i64, _f32, _f64, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_size_t


class QknrLayout(ctypes.Structure):
    """Token strides (elements) of each tensor, and the optional K slot map
    with the row count of the K output it indexes."""
    _fields_ = [("q_stride", ctypes.c_int64), ("k_stride", ctypes.c_int64),
                ("q_out_stride", ctypes.c_int64), ("k_out_stride", ctypes.c_int64),
                ("dq_out_stride", ctypes.c_int64), ("dk_out_stride", ctypes.c_int64),
                ("k_out_slots", ctypes.c_void_p), ("k_out_rows", ctypes.c_int64)]


class QknrOptions(ctypes.Structure):
    """Flags, layout, biases, frequency table and attention factor of
    qknr_fwd_opt / qknr_bwd_opt."""
    _fields_ = [("flags", ctypes.c_uint32), ("layout", ctypes.POINTER(QknrLayout)),
                ("bq", ctypes.c_void_p), ("bk", ctypes.c_void_p),
                ("inv_freq", ctypes.POINTER(ctypes.c_double)),
                ("attention_factor", ctypes.c_double),
                ("norm_group_q", ctypes.c_int32), ("norm_group_k", ctypes.c_int32)]


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
    L.qknr_bwd_noalloc.restype = ctypes.c_int
    L.qknr_bwd_noalloc.argtypes = [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64,
                                   _i32, _i32, _i32, _i32, _f32, _f64, ctypes.c_int, _c_void_p,
                                   _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                   _c_void_p]
    L.qknr_fwd_ex.restype = ctypes.c_int
    L.qknr_fwd_ex.argtypes = [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i32,
                              _i32, _i32, _i32, _f32, _f64, ctypes.c_int, ctypes.c_uint32,
                              ctypes.POINTER(QknrLayout), _c_void_p, _c_void_p, _c_void_p]
    L.qknr_bwd_ex.restype = ctypes.c_int
    L.qknr_bwd_ex.argtypes = [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i32,
                              _i32, _i32, _i32, _f32, _f64, ctypes.c_int, ctypes.c_uint32,
                              ctypes.POINTER(QknrLayout), _c_void_p, _c_void_p, _c_void_p,
                              _c_void_p, _c_void_p, _c_void_p, _c_void_p, _sz, _c_void_p]
    L.qknr_fwd_opt.restype = ctypes.c_int
    L.qknr_fwd_opt.argtypes = [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i32,
                               _i32, _i32, _i32, _f32, _f64, ctypes.c_int,
                               ctypes.POINTER(QknrOptions), _c_void_p, _c_void_p, _c_void_p]
    L.qknr_bwd_opt.restype = ctypes.c_int
    L.qknr_bwd_opt.argtypes = [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i32,
                               _i32, _i32, _i32, _f32, _f64, ctypes.c_int,
                               ctypes.POINTER(QknrOptions), _c_void_p, _c_void_p, _c_void_p,
                               _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                               _sz, _c_void_p]
    L.qknr_bwd_opt_workspace_bytes.restype = _sz
    L.qknr_bwd_opt_workspace_bytes.argtypes = [_i64, _i32, _i32, _i32, _i32, ctypes.c_int,
                                               ctypes.POINTER(QknrOptions)]
    L.qknr_bfd_workspace_bytes.restype = _sz
    L.qknr_bfd_workspace_bytes.argtypes = [_i32, _i32]
    L.qknr_bfd_pack.restype = ctypes.c_int
    L.qknr_bfd_pack.argtypes = [_c_void_p, _i32, _i32, _i32, _c_void_p, _c_void_p, _c_void_p,
                                _c_void_p, _c_void_p, _c_void_p, _sz, _c_void_p]
    L.qknr_bwd_workspace_bytes.restype = _sz
    L.qknr_bwd_workspace_bytes.argtypes = [_i64, _i32, _i32, _i32, ctypes.c_int]
    L.qknr_status_string.restype = ctypes.c_char_p
    L.qknr_status_string.argtypes = [ctypes.c_int]
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


def qknr_bwd_noalloc(q, k, wq, wk, position_ids, dq_out, dk_out, rotary_dim: int, eps: float,
                     theta: float, dq, dk, dwq, dwk, stream=None):
    """qknr_bwd into caller-provided outputs with no workspace: the library keeps
    the weight-gradient partials in its own static device array, so neither the
    library nor this binding allocates device memory (position_ids must already
    be int32).  Calls that overlap on one GPU race.  Returns (dq, dk, dwq, dwk)."""
    T, hq, hkv, D = _shapes(q, k)
    dev = q.device
    dt = q.dtype
    for n, t, s in (("q", q, (T, hq, D)), ("k", k, (T, hkv, D)), ("wq", wq, (D,)), ("wk", wk, (D,)),
                    ("dq_out", dq_out, (T, hq, D)), ("dk_out", dk_out, (T, hkv, D)),
                    ("dq", dq, (T, hq, D)), ("dk", dk, (T, hkv, D)), ("dwq", dwq, (D,)),
                    ("dwk", dwk, (D,))):
        _check(n, t, dt, s, dev)
    _check("position_ids", position_ids, torch.int32, (T,), dev)
    st = lib.qknr_bwd_noalloc(q.data_ptr(), k.data_ptr(), wq.data_ptr(), wk.data_ptr(),
                              position_ids.data_ptr(), T, hq, hkv, D, int(rotary_dim), float(eps),
                              float(theta), _dtype_code(q), dq_out.data_ptr(), dk_out.data_ptr(),
                              dq.data_ptr(), dk.data_ptr(), dwq.data_ptr(), dwk.data_ptr(),
                              _stream(dev, stream))
    if st != 0:
        raise QknrError(st, "qknr_bwd_noalloc")
    return dq, dk, dwq, dwk


# ---- extended entry points: strided views, paged K output, convention flags ----

def _token_stride(name, t, dtype, tokens, heads, D, device):
    """Token stride (elements) of a [tokens, heads, D] view whose heads are
    contiguous; the library checks the stride's size and alignment."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if t.dim() != 3 or (tokens is not None and t.shape[0] != tokens) or tuple(t.shape[1:]) != (heads, D):
        raise ValueError("%s has shape %s, expected [%s, %d, %d]"
                         % (name, tuple(t.shape), "tokens" if tokens is None else tokens, heads, D))
    if t.stride(2) != 1 or t.stride(1) != D:
        raise ValueError("%s must have contiguous heads (strides [*, %d, 1]), got %s"
                         % (name, D, t.stride()))
    return t.stride(0) if t.shape[0] > 1 else heads * D


def _weights(wq, wk, flags, dt, D, dev, hq=1, hkv=1):
    if flags & QKNR_FLAG_NO_WEIGHT:
        return 0, 0
    for n, t, shape in zip(("wq", "wk"), (wq, wk), _wshapes(flags, hq, hkv, D)):
        _check(n, t, dt, shape, dev)
    return wq.data_ptr(), wk.data_ptr()


def qknr_fwd_ex(q, k, wq, wk, position_ids, rotary_dim: int, eps: float, theta: float,
                flags: int = 0, q_out=None, k_out=None, k_out_slots=None, stream=None):
    """Forward on [tokens, heads, D] views with any token stride (e.g. slices
    of a fused QKV projection), writing q_out/k_out (dense new tensors if None;
    pass q_out=q, k_out=k for in place).  k_out_slots (int64 [tokens]) writes
    token t's K heads at row k_out_slots[t] of k_out (a slot outside
    [0, k_out.shape[0]) is skipped), for a KV cache viewed as [slots, hkv, D].  wq/wk may be None with
    QKNR_FLAG_NO_WEIGHT.  Returns (q_out, k_out)."""
    if q.dim() != 3 or k.dim() != 3 or q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2]:
        raise ValueError("q must be [tokens, hq, D] and k [tokens, hkv, D]")
    T, hq, D = q.shape
    hkv = k.shape[1]
    dev, dt = q.device, q.dtype
    lay = QknrLayout()
    lay.q_stride = _token_stride("q", q, dt, T, hq, D, dev)
    lay.k_stride = _token_stride("k", k, dt, T, hkv, D, dev)
    pw = _weights(wq, wk, flags, dt, D, dev)
    pos = _positions(position_ids, T, dev)
    q_out = torch.empty((T, hq, D), dtype=dt, device=dev) if q_out is None else q_out
    if k_out is None:
        if k_out_slots is not None:
            raise ValueError("k_out_slots needs the k_out buffer the slots index")
        k_out = torch.empty((T, hkv, D), dtype=dt, device=dev)
    lay.q_out_stride = _token_stride("q_out", q_out, dt, T, hq, D, dev)
    lay.k_out_stride = _token_stride("k_out", k_out, dt, None if k_out_slots is not None else T,
                                     hkv, D, dev)
    lay.dq_out_stride, lay.dk_out_stride = hq * D, hkv * D
    if k_out_slots is not None:
        _check("k_out_slots", k_out_slots, torch.int64, (T,), dev)
        lay.k_out_slots = k_out_slots.data_ptr()
        lay.k_out_rows = int(k_out.shape[0])  # slots outside [0, rows) are not written
    st = lib.qknr_fwd_ex(q.data_ptr(), k.data_ptr(), pw[0], pw[1], pos.data_ptr(), T, hq, hkv, D,
                         int(rotary_dim), float(eps), float(theta), _dtype_code(q), int(flags),
                         ctypes.byref(lay), q_out.data_ptr(), k_out.data_ptr(), _stream(dev, stream))
    if st != 0:
        raise QknrError(st, "qknr_fwd_ex")
    return q_out, k_out


def qknr_bwd_ex(q, k, wq, wk, position_ids, dq_out, dk_out, rotary_dim: int, eps: float,
                theta: float, flags: int = 0, dq=None, dk=None, dwq=None, dwk=None,
                workspace=None, stream=None):
    """Backward of qknr_fwd_ex (same flags) on strided [tokens, heads, D] views.
    Returns (dq, dk, dwq, dwk); dwq/dwk are None with QKNR_FLAG_NO_WEIGHT."""
    if q.dim() != 3 or k.dim() != 3 or q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2]:
        raise ValueError("q must be [tokens, hq, D] and k [tokens, hkv, D]")
    T, hq, D = q.shape
    hkv = k.shape[1]
    dev, dt = q.device, q.dtype
    lay = QknrLayout()
    lay.q_stride = _token_stride("q", q, dt, T, hq, D, dev)
    lay.k_stride = _token_stride("k", k, dt, T, hkv, D, dev)
    lay.dq_out_stride = _token_stride("dq_out", dq_out, dt, T, hq, D, dev)
    lay.dk_out_stride = _token_stride("dk_out", dk_out, dt, T, hkv, D, dev)
    pw = _weights(wq, wk, flags, dt, D, dev)
    pos = _positions(position_ids, T, dev)
    dq = torch.empty((T, hq, D), dtype=dt, device=dev) if dq is None else dq
    dk = torch.empty((T, hkv, D), dtype=dt, device=dev) if dk is None else dk
    lay.q_out_stride = _token_stride("dq", dq, dt, T, hq, D, dev)
    lay.k_out_stride = _token_stride("dk", dk, dt, T, hkv, D, dev)
    if flags & QKNR_FLAG_NO_WEIGHT:
        dwq = dwk = None
        pdw = (0, 0)
    else:
        dwq = torch.empty((D,), dtype=dt, device=dev) if dwq is None else dwq
        dwk = torch.empty((D,), dtype=dt, device=dev) if dwk is None else dwk
        _check("dwq", dwq, dt, (D,), dev)
        _check("dwk", dwk, dt, (D,), dev)
        pdw = (dwq.data_ptr(), dwk.data_ptr())
    need = qknr_bwd_workspace_bytes(T, hq, hkv, D, _dtype_code(q))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on %s" % dev)
    wbytes = workspace.numel() * workspace.element_size()
    st = lib.qknr_bwd_ex(q.data_ptr(), k.data_ptr(), pw[0], pw[1], pos.data_ptr(), T, hq, hkv, D,
                         int(rotary_dim), float(eps), float(theta), _dtype_code(q), int(flags),
                         ctypes.byref(lay), dq_out.data_ptr(), dk_out.data_ptr(), dq.data_ptr(),
                         dk.data_ptr(), pdw[0], pdw[1], workspace.data_ptr(), wbytes,
                         _stream(dev, stream))
    if st != 0:
        raise QknrError(st, "qknr_bwd_ex")
    return dq, dk, dwq, dwk


# ---- entry points with every option: biases, frequency table, attention factor ----

def _wshapes(flags, hq, hkv, D):
    """Shapes of (wq, wk): [D] each, or [H, D] with QKNR_FLAG_HEAD_WEIGHTS."""
    if flags & QKNR_FLAG_HEAD_WEIGHTS:
        return (hq, D), (hkv, D)
    return (D,), (D,)


def _options(flags, lay, bq, bk, inv_freq, attention_factor, rotary_dim, dt, D, dev,
             norm_groups=None, hq=1, hkv=1):
    """Fill a QknrOptions; returns it with the objects it points into (kept
    alive by the caller for the duration of the call)."""
    opt = QknrOptions()
    opt.flags = int(flags)
    opt.layout = ctypes.pointer(lay)
    if (bq is None) != (bk is None):
        raise ValueError("pass both biases or neither")
    if bq is not None:
        sq, sk = _wshapes(flags, hq, hkv, D)
        _check("bq", bq, dt, sq, dev)
        _check("bk", bk, dt, sk, dev)
        opt.bq, opt.bk = bq.data_ptr(), bk.data_ptr()
    if norm_groups is not None:
        opt.norm_group_q, opt.norm_group_k = (int(g) for g in norm_groups)
    tab = None
    if inv_freq is not None:
        vals = [float(v) for v in (inv_freq.tolist() if hasattr(inv_freq, "tolist") else inv_freq)]
        if len(vals) != rotary_dim // 2:
            raise ValueError("inv_freq must hold rotary_dim/2 = %d values" % (rotary_dim // 2))
        tab = (ctypes.c_double * max(1, len(vals)))(*vals)
        opt.inv_freq = ctypes.cast(tab, ctypes.POINTER(ctypes.c_double))
    opt.attention_factor = float(attention_factor)
    return opt, (lay, tab)


def qknr_fwd_opt(q, k, wq, wk, position_ids, rotary_dim: int, eps: float, theta: float,
                 flags: int = 0, bq=None, bk=None, inv_freq=None, attention_factor: float = 1.0,
                 q_out=None, k_out=None, k_out_slots=None, norm_groups=None, stream=None):
    """qknr_fwd_ex plus QK-LayerNorm (flag), biases added after the weight, a
    frequency table (rotary_dim/2 values, host sequence or tensor) replacing
    theta^(-2i/d), an attention factor on cos and sin, norm groups
    (gq, gk) of heads sharing one inverse RMS, and [H, D] weights and biases
    with QKNR_FLAG_HEAD_WEIGHTS.  Returns (q_out, k_out)."""
    if q.dim() != 3 or k.dim() != 3 or q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2]:
        raise ValueError("q must be [tokens, hq, D] and k [tokens, hkv, D]")
    T, hq, D = q.shape
    hkv = k.shape[1]
    dev, dt = q.device, q.dtype
    lay = QknrLayout()
    lay.q_stride = _token_stride("q", q, dt, T, hq, D, dev)
    lay.k_stride = _token_stride("k", k, dt, T, hkv, D, dev)
    pw = _weights(wq, wk, flags, dt, D, dev, hq, hkv)
    pos = _positions(position_ids, T, dev)
    q_out = torch.empty((T, hq, D), dtype=dt, device=dev) if q_out is None else q_out
    if k_out is None:
        if k_out_slots is not None:
            raise ValueError("k_out_slots needs the k_out buffer the slots index")
        k_out = torch.empty((T, hkv, D), dtype=dt, device=dev)
    lay.q_out_stride = _token_stride("q_out", q_out, dt, T, hq, D, dev)
    lay.k_out_stride = _token_stride("k_out", k_out, dt, None if k_out_slots is not None else T,
                                     hkv, D, dev)
    lay.dq_out_stride, lay.dk_out_stride = hq * D, hkv * D
    if k_out_slots is not None:
        _check("k_out_slots", k_out_slots, torch.int64, (T,), dev)
        lay.k_out_slots = k_out_slots.data_ptr()
        lay.k_out_rows = int(k_out.shape[0])  # slots outside [0, rows) are not written
    opt, keep = _options(flags, lay, bq, bk, inv_freq, attention_factor, rotary_dim, dt, D, dev,
                         norm_groups, hq, hkv)
    st = lib.qknr_fwd_opt(q.data_ptr(), k.data_ptr(), pw[0], pw[1], pos.data_ptr(), T, hq, hkv, D,
                          int(rotary_dim), float(eps), float(theta), _dtype_code(q),
                          ctypes.byref(opt), q_out.data_ptr(), k_out.data_ptr(),
                          _stream(dev, stream))
    del keep
    if st != 0:
        raise QknrError(st, "qknr_fwd_opt")
    return q_out, k_out


def qknr_bwd_opt(q, k, wq, wk, position_ids, dq_out, dk_out, rotary_dim: int, eps: float,
                 theta: float, flags: int = 0, bias_grads: bool = False, inv_freq=None,
                 attention_factor: float = 1.0, dq=None, dk=None, dwq=None, dwk=None, dbq=None,
                 dbk=None, workspace=None, norm_groups=None, stream=None):
    """Backward of qknr_fwd_opt (same flags, table, factor and norm groups;
    the biases do not enter it).  Returns (dq, dk, dwq, dwk, dbq, dbk), the
    weight and bias gradients shaped like the weights; dwq/dwk are None with
    QKNR_FLAG_NO_WEIGHT and dbq/dbk None unless bias_grads."""
    if q.dim() != 3 or k.dim() != 3 or q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2]:
        raise ValueError("q must be [tokens, hq, D] and k [tokens, hkv, D]")
    T, hq, D = q.shape
    hkv = k.shape[1]
    dev, dt = q.device, q.dtype
    lay = QknrLayout()
    lay.q_stride = _token_stride("q", q, dt, T, hq, D, dev)
    lay.k_stride = _token_stride("k", k, dt, T, hkv, D, dev)
    lay.dq_out_stride = _token_stride("dq_out", dq_out, dt, T, hq, D, dev)
    lay.dk_out_stride = _token_stride("dk_out", dk_out, dt, T, hkv, D, dev)
    pw = _weights(wq, wk, flags, dt, D, dev, hq, hkv)
    pos = _positions(position_ids, T, dev)
    dq = torch.empty((T, hq, D), dtype=dt, device=dev) if dq is None else dq
    dk = torch.empty((T, hkv, D), dtype=dt, device=dev) if dk is None else dk
    lay.q_out_stride = _token_stride("dq", dq, dt, T, hq, D, dev)
    lay.k_out_stride = _token_stride("dk", dk, dt, T, hkv, D, dev)
    sq, sk = _wshapes(flags, hq, hkv, D)
    grads = []
    for want, a, b, na, nb in ((not flags & QKNR_FLAG_NO_WEIGHT, dwq, dwk, "dwq", "dwk"),
                               (bias_grads, dbq, dbk, "dbq", "dbk")):
        if not want:
            grads += [None, None]
            continue
        a = torch.empty(sq, dtype=dt, device=dev) if a is None else a
        b = torch.empty(sk, dtype=dt, device=dev) if b is None else b
        _check(na, a, dt, sq, dev)
        _check(nb, b, dt, sk, dev)
        grads += [a, b]
    ptrs = [0 if t is None else t.data_ptr() for t in grads]
    opt, keep = _options(flags, lay, None, None, inv_freq, attention_factor, rotary_dim, dt, D, dev,
                         norm_groups, hq, hkv)
    need = int(lib.qknr_bwd_opt_workspace_bytes(T, hq, hkv, D, int(rotary_dim), _dtype_code(q),
                                                ctypes.byref(opt)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on %s" % dev)
    wbytes = workspace.numel() * workspace.element_size()
    st = lib.qknr_bwd_opt(q.data_ptr(), k.data_ptr(), pw[0], pw[1], pos.data_ptr(), T, hq, hkv, D,
                          int(rotary_dim), float(eps), float(theta), _dtype_code(q),
                          ctypes.byref(opt), dq_out.data_ptr(), dk_out.data_ptr(), dq.data_ptr(),
                          dk.data_ptr(), ptrs[0], ptrs[1], ptrs[2], ptrs[3], workspace.data_ptr(),
                          wbytes, _stream(dev, stream))
    del keep
    if st != 0:
        raise QknrError(st, "qknr_bwd_opt")
    return (dq, dk) + tuple(grads)


def qknr_bwd_opt_workspace_bytes(tokens: int, hq: int, hkv: int, head_dim: int, rotary_dim: int,
                                 dtype, flags: int = 0, norm_groups=None) -> int:
    """Workspace bytes of qknr_bwd_opt for these sizes, flags and norm groups."""
    code = dtype if isinstance(dtype, int) else (QKNR_BF16 if dtype == torch.bfloat16 else QKNR_F32)
    opt = QknrOptions()
    opt.flags = int(flags)
    if norm_groups is not None:
        opt.norm_group_q, opt.norm_group_k = (int(g) for g in norm_groups)
    return int(lib.qknr_bwd_opt_workspace_bytes(int(tokens), int(hq), int(hkv), int(head_dim),
                                                int(rotary_dim), code, ctypes.byref(opt)))


def qknr_bfd_pack(lengths, capacity: int, max_bins: int, workspace=None, stream=None):
    """Best-Fit-Decreasing packing on the device of int32 document lengths
    (a CUDA tensor) into buffers of `capacity` tokens.  Returns a dict of device
    tensors: doc_start [n], position_ids [max_bins * capacity] (valid for the
    first bins * capacity tokens), cu_seqlens [n + max_bins + 1] (valid for
    segments + 1 entries), counts [2] = {bins, segments}, status [1]; read
    counts and status after synchronising."""
    if not isinstance(lengths, torch.Tensor) or lengths.dtype != torch.int32 or lengths.dim() != 1:
        raise TypeError("lengths must be a 1-D int32 tensor")
    if not lengths.is_contiguous():
        raise ValueError("lengths must be contiguous")
    dev = lengths.device
    n = int(lengths.shape[0])
    i32 = dict(dtype=torch.int32, device=dev)
    out = dict(doc_start=torch.empty(max(n, 1), **i32),
               position_ids=torch.empty(max(1, int(max_bins) * int(capacity)), **i32),
               cu_seqlens=torch.empty(n + int(max_bins) + 1, **i32),
               counts=torch.empty(2, **i32), status=torch.empty(1, **i32))
    need = int(lib.qknr_bfd_workspace_bytes(n, int(max_bins)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    wbytes = workspace.numel() * workspace.element_size()
    st = lib.qknr_bfd_pack(lengths.data_ptr() if n else None, n, int(capacity), int(max_bins),
                           out["doc_start"].data_ptr(), out["position_ids"].data_ptr(),
                           out["cu_seqlens"].data_ptr(), out["counts"].data_ptr(),
                           out["status"].data_ptr(), workspace.data_ptr(), wbytes,
                           _stream(dev, stream))
    if st != 0:
        raise QknrError(st, "qknr_bfd_pack")
    out["doc_start"] = out["doc_start"][:n]
    return out

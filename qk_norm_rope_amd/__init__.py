"""Fused per-head QK-Norm + RoPE for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libqknr.so`` (declared in
``include/qknr.h``).  Every step of the operation runs in the library's HIP
kernels; this module only checks tensor metadata, allocates outputs with torch
(device memory and streams are torch's) and passes raw pointers and the current
HIP stream.  There is no fallback: if the library is not built, importing the
binding's entry points raises.
"""

from ._lib import (  # noqa: F401
    QKNR_BF16,
    QKNR_F32,
    QKNR_FLAG_FREQ_HEAD_DIM,
    QKNR_FLAG_HEAD_WEIGHTS,
    QKNR_FLAG_INTERLEAVED,
    QKNR_FLAG_LAYERNORM,
    QKNR_FLAG_NO_WEIGHT,
    QknrError,
    QknrLayout,
    QknrOptions,
    lib,
    lib_path,
    qknr_bfd_pack,
    qknr_bwd,
    qknr_bwd_ex,
    qknr_bwd_noalloc,
    qknr_bwd_opt,
    qknr_bwd_opt_workspace_bytes,
    qknr_bwd_workspace_bytes,
    qknr_fwd,
    qknr_fwd_ex,
    qknr_fwd_opt,
    qknr_status_string,
)

"""Shared test helpers: moving stored inputs to the GPU, and the parity rules
(oracle/parity.py, re-exported here).

Parity rules (tolerances):
  * fp32 I/O: max |gpu - oracle| <= 2e-5 against the unrounded fp64 oracle value.
    A weight gradient is a sum over every row of its tensor, so its size (and
    the rounding of an fp32 sum) grows with the row count: for it the bound is
    2e-5 * max(1, RMS of the oracle's [D] vector), the fp32 counterpart of the
    whole-vector floor of the bf16 rule.
  * bf16 I/O: o = one-step round-to-nearest-even of the fp64 oracle value to
    bf16; ulp(o) = 2^(floor(log2|o|) - 7) (2^-133 below 2^-126).  An element
    passes iff |v - o| <= 2 * max(ulp(o), 2^-16 * rms_row), rms_row being the
    RMS of the oracle's fp64 output over that element's row (for dw: over the
    whole [D] vector).  The floor covers outputs near zero where terms cancel
    and an fp32 pipeline cannot reach 2 ulp of a tiny value; the count of
    elements beyond a strict 2 ulp is reported as well.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle

from oracle.parity import (  # noqa: F401  (the rules, re-exported for the tests)
    F32_TOL,
    bf16_ulp_bits,
    brief,
    compare,
    merge_stats,
)


def to_device(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)


def to_host_bits(t: torch.Tensor, dtype: str) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def gpu_values(t: torch.Tensor, dtype: str) -> np.ndarray:
    """GPU result widened exactly to fp64."""
    return oracle.decode(to_host_bits(t, dtype), dtype)



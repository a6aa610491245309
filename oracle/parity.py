"""Parity rules: how a GPU result is compared with the fp64 oracle (test
infrastructure, used by the tests and the benchmark's CPU-baseline leg).

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

from . import bf16_bits_to_f64, round_bf16

F32_TOL = 2e-5


def bf16_ulp_bits(bits: np.ndarray) -> np.ndarray:
    """ulp of bf16 values given their bit patterns: 2^(e - 127 - 7) for a
    biased exponent e >= 1, 2^-133 for zero and subnormals."""
    e = ((np.asarray(bits, np.uint16) >> np.uint16(7)) & np.uint16(0xFF)).astype(np.int32)
    return np.ldexp(1.0, np.maximum(e, 1) - 134)


def compare(got: np.ndarray, want64: np.ndarray, dtype: str, what: str = "", row_axis=-1,
            row_sum: bool = False) -> dict:
    """Compare GPU values (fp64-widened) with fp64 oracle values; raises on
    failure, returns statistics.  row_sum marks a weight gradient (a sum over
    rows), whose fp32 bound scales with the vector's RMS."""
    got = np.asarray(got, np.float64)
    want64 = np.asarray(want64, np.float64)
    assert got.shape == want64.shape, (what, got.shape, want64.shape)
    if got.size == 0:
        return {"n": 0}
    if not np.all(np.isfinite(got)):
        raise AssertionError("%s: non-finite GPU output" % what)
    if dtype == "f32":
        err = np.abs(got - want64)
        m = float(err.max())
        tol = F32_TOL
        if row_sum:
            tol *= max(1.0, float(np.sqrt(np.mean(want64 * want64))))
        if m > tol:
            i = np.unravel_index(int(err.argmax()), err.shape)
            raise AssertionError("%s: max abs err %.3g > %.3g at %s (gpu %r, oracle %r)"
                                 % (what, m, tol, i, got[i], want64[i]))
        return {"n": got.size, "max_abs": m, "tol": tol}
    ob = round_bf16(want64)
    o = bf16_bits_to_f64(ob)
    ulp = bf16_ulp_bits(ob)
    rms = np.sqrt(np.mean(want64 * want64, axis=row_axis, keepdims=True)) if want64.ndim else np.abs(want64)
    floor = np.broadcast_to(2.0 ** -16 * rms, o.shape)
    err = np.abs(got - o)
    allow = 2.0 * np.maximum(ulp, floor)
    bad = err > allow
    strict = int(np.count_nonzero(err > 2.0 * ulp))
    stats = {"n": got.size, "max_abs": float(err.max()), "max_ulp": float((err / ulp).max()),
             "beyond_strict_2ulp": strict, "exact": int(np.count_nonzero(err == 0))}
    if bad.any():
        i = np.unravel_index(int(np.argmax(bad)), bad.shape)
        raise AssertionError("%s: %d of %d elements beyond tolerance; first at %s: gpu %r, oracle "
                             "rounded %r (fp64 %r), allowed %r; stats %s"
                             % (what, int(bad.sum()), got.size, i, got[i], o[i], want64[i],
                                allow[i], stats))
    return stats


def merge_stats(acc: dict | None, st: dict) -> dict:
    """Combine the statistics of compare() over chunks of one tensor."""
    if acc is None:
        return dict(st)
    out = dict(acc)
    out["n"] = acc.get("n", 0) + st.get("n", 0)
    for key in ("max_abs", "max_ulp"):
        if key in st:
            out[key] = max(acc.get(key, 0.0), st[key])
    for key in ("beyond_strict_2ulp", "exact"):
        if key in st:
            out[key] = acc.get(key, 0) + st[key]
    return out


def brief(stats: dict) -> dict:
    """The statistics worth printing: elements, max abs and ulp error, and the
    count beyond a strict 2 ulp (bf16)."""
    keys = ("n", "max_abs", "max_ulp", "beyond_strict_2ulp")
    return {k: (float("%.3g" % v) if isinstance(v, float) else v) for k, v in stats.items()
            if k in keys}

"""Best-Fit-Decreasing sequence packing for the packed-sequence workload.

Chronicals ("Chronicals: A High-Performance Framework for LLM Fine-Tuning with
3.51x Speedup over Unsloth", abstract, contribution (4)) packs documents into
fixed-length buffers with Best-Fit Decreasing to avoid padding; position ids
then restart at 0 at every document boundary inside a buffer.  This module
builds such a buffer from document lengths drawn log-uniformly.

Tie-breaks (the pages give none): documents are sorted by length, longest
first, ties kept in draw order; each goes into the open bin whose remaining
capacity is smallest among those it fits (ties: lowest bin index), else into a
new bin.  The fullest bin (ties: lowest index) is the buffer; if it is not full,
one filler document of the remaining length completes it.
"""

from __future__ import annotations

import numpy as np


def draw_lengths(g: np.random.Generator, lo: int, hi: int, pool_tokens: int,
                 batch: int = 256) -> np.ndarray:
    """Lengths clip(round(exp(U[ln lo, ln hi])), lo, hi), drawn until their sum
    reaches ``pool_tokens``."""
    out = []
    total = 0
    while total < pool_tokens:
        u = g.uniform(np.log(lo), np.log(hi), size=batch)
        L = np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int64)
        for x in L:
            out.append(int(x))
            total += int(x)
            if total >= pool_tokens:
                break
    return np.asarray(out, np.int64)


def bfd_bins(lengths: np.ndarray, capacity: int):
    """Best-Fit-Decreasing packing; returns a list of bins, each a list of
    document lengths in placement order."""
    lengths = np.asarray(lengths, np.int64)
    if np.any(lengths <= 0) or np.any(lengths > capacity):
        raise ValueError("document lengths must lie in [1, capacity]")
    order = np.argsort(-lengths, kind="stable")
    bins: list[list[int]] = []
    free: list[int] = []
    for i in order:
        L = int(lengths[i])
        best = -1
        for b, f in enumerate(free):
            if f >= L and (best < 0 or f < free[best]):
                best = b
        if best < 0:
            bins.append([L])
            free.append(capacity - L)
        else:
            bins[best].append(L)
            free[best] -= L
    return bins


def pack_one_buffer(lengths: np.ndarray, capacity: int) -> list[int]:
    """Document lengths of one full buffer of ``capacity`` tokens: the fullest
    BFD bin, completed by a filler document if it is not full."""
    bins = bfd_bins(lengths, capacity)
    fill = [sum(b) for b in bins]
    best = int(np.argmax(fill))  # argmax returns the lowest index among ties
    docs = list(bins[best])
    rem = capacity - fill[best]
    if rem > 0:
        docs.append(rem)
    return docs

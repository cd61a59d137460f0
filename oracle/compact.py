"""Compaction of kept rows -- oracle (test infrastructure only).

Random Attention, Appendix F ("Engine details"): after each eviction the KV
tensors are compacted with a gather, keep-sets sorted chronologically. Row r
of the output is row kept[r] of the input, for K, V and the positions
(slot index when no position array is given).

``compact_holes`` is the in-place alternative the pages' engine notes leave
open: the n_kept kept rows end up in slots 0..n_kept-1 as with the gather,
but a kept row already below n_kept stays where it is, and each kept row at
or above n_kept moves into a hole (an evicted slot below n_kept); the i-th
such row in slot order fills the i-th hole in slot order. Slot order is then
no longer chronological, so positions travel with the rows.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def compact(K: np.ndarray, V: np.ndarray, pos: Optional[np.ndarray], kept) -> tuple:
    """(K[kept], V[kept], pos[kept] or kept) for one head; K, V are (T, d) arrays."""
    idx = np.asarray(kept, dtype=np.int64)
    if idx.size and (idx.min() < 0 or idx.max() >= K.shape[0]):
        raise IndexError("kept index out of range")
    p = idx.astype(np.int32) if pos is None else np.asarray(pos)[idx].astype(np.int32)
    return np.asarray(K)[idx], np.asarray(V)[idx], p


def compact_holes(K: np.ndarray, V: np.ndarray, pos: Optional[np.ndarray], kept) -> tuple:
    """In-place hole filling for one head: (K', V', pos', moves) with n_kept rows.

    K, V are the head's (T, d) rows; ``moves`` lists the (source, destination) slot pairs.
    """
    idx = sorted(int(x) for x in kept)
    n = len(idx)
    T = np.asarray(K).shape[0]
    if n and (idx[0] < 0 or idx[-1] >= T):
        raise IndexError("kept index out of range")
    kept_set = set(idx)
    holes = [x for x in range(n) if x not in kept_set]
    movers = [x for x in idx if x >= n]
    assert len(holes) == len(movers)
    Kc, Vc = np.array(K, copy=True), np.array(V, copy=True)
    pc = np.arange(T, dtype=np.int32) if pos is None else np.array(pos, dtype=np.int32, copy=True)
    for src, dst in zip(movers, holes):
        Kc[dst], Vc[dst], pc[dst] = Kc[src], Vc[src], pc[src]
    return Kc[:n], Vc[:n], pc[:n], list(zip(movers, holes))

"""Gather-compaction of kept rows -- oracle (test infrastructure only).

Random Attention, Appendix F ("Engine details"): after each eviction the KV
tensors are compacted with a gather, keep-sets sorted chronologically. Row r
of the output is row kept[r] of the input, for K, V and the positions
(slot index when no position array is given).
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

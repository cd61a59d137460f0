"""Pinning, top-n selection and random selection -- oracle (test infrastructure only).

Sources:
  * TriAttention summary, section 3.4 "KV Cache Pruning Procedure": when the
    cache exceeds the budget B, keys are ranked by score and the top B are
    kept; the rest are evicted for good.
  * TriAttention blog, inference-time scoring step: prefill (prompt) tokens
    are always kept by default and only decode tokens compete for what
    remains of the budget.
  * Random Attention, section 2 ("Periodic eviction with budget K and buffer
    r"): a buffer of the most recent pairs is never scored, the candidates
    are the cached positions outside it, and the top-K candidates are kept
    (Eq. 2).
  * Random Attention, section 3: the prompt is never evicted; every other
    candidate gets an i.i.d. Uniform(0,1) score drawn independently per KV
    head at every eviction (Eq. 3, Algorithm 1).
  * Random Attention, Appendix F: keep-sets are sorted chronologically before
    compaction.
  * Random Attention, section 4.1 (the recency+prompt diagnostic: keep the
    prompt and fill the rest with the contiguous recent window) and sections
    5.2-5.3 (the shared-draw control: one random keep-set used by every head).
  * TriAttention blog, eviction step (union-based selection: each head picks
    its own top-k, the union is formed, the final set is taken from the union
    by a combined score and topped up by score order when the union is short).

Readings taken where the pages leave a step open (each is also listed with
the design notes):
  * B counts every kept entry: prompt + recent window + selected.
  * If T <= B nothing is compressed: kept = 0..T-1.
  * The prompt is a hard pin: if P >= B, kept = the whole prompt, nothing is
    selected and the recent window is dropped (n_kept = P).
  * The recent window is a soft pin clipped to R' = min(R, B - P, T - P) and
    holds the latest R' slots, so |kept| = B whenever P <= B.
  * Ranking is (score descending, slot ascending); NaN ranks as -inf and
    -0.0 equals +0.0.
  * The random score of a candidate slot j is word (p_j mod 4) of
    Philox4x32-10 with counter (p_j div 4, (layer << 16) | head, seq, event)
    and key (seed mod 2^32, seed >> 32), read as the uniform u = word / 2^32;
    ties go to the lower slot.
  * Recency+prompt keeps the prompt and the n_kept - P latest slots (the
    evictable range's n_sel latest slots joined to the recent window).
  * The shared draw is the draw of layer 0, KV head 0, used by every
    (layer, KV head) of the sequence.
  * Union-based selection works per KV head over its G query heads, ranks
    each query head's evictable slots by its own score, takes per-head top-k
    (k = ceil(n_sel / G) unless given), and ranks by the combined score
    (slot ascending on ties) both inside the union and for the top-up.
"""
from __future__ import annotations

from typing import NamedTuple, Optional

import numpy as np

from .philox import philox4x32_10_np


class Partition(NamedTuple):
    T: int          # cached slots
    P: int          # pinned prompt slots [0, P)
    R: int          # pinned recent slots [T - R, T)
    e_lo: int       # evictable range [e_lo, e_hi)
    e_hi: int
    n_sel: int      # slots selected from the evictable range
    n_kept: int     # |kept|
    compress: bool  # False when T <= B (kept = everything)


def partition(T: int, P: int, B: int, R: int) -> Partition:
    """Split a head's T slots into prompt, recent window and evictable range."""
    T = max(int(T), 0)
    P = min(max(int(P), 0), T)
    B, R = int(B), max(int(R), 0)
    if B < 1:
        raise ValueError("budget must be >= 1")
    if T <= B:
        return Partition(T, P, 0, P, P, 0, T, False)
    R_eff = min(R, max(0, B - P), T - P)
    e_lo, e_hi = P, T - R_eff
    n_sel = max(0, B - P - R_eff)
    n_kept = max(B, P)
    return Partition(T, P, R_eff, e_lo, e_hi, n_sel, n_kept, True)


def canonical_scores(scores) -> np.ndarray:
    """fp64 copy with NaN -> -inf and -0.0 -> +0.0 (exact upcast otherwise)."""
    s = np.array(scores, dtype=np.float64, copy=True)
    s[np.isnan(s)] = -np.inf
    s[s == 0.0] = 0.0
    return s


def _assemble(part: Partition, selected: np.ndarray) -> np.ndarray:
    pins = np.concatenate([np.arange(0, part.P), np.arange(part.T - part.R, part.T)])
    kept = np.sort(np.concatenate([pins, np.asarray(selected, dtype=np.int64)]))
    assert kept.size == part.n_kept
    return kept.astype(np.int32)


def _top_by_rank(values: np.ndarray, part: Partition) -> np.ndarray:
    """The n_sel evictable slots ranked first by (value desc, slot asc)."""
    slots = np.arange(part.e_lo, part.e_hi, dtype=np.int64)
    v = values[part.e_lo:part.e_hi]
    order = np.lexsort((slots, -v))          # primary key: -v ascending; secondary: slot ascending
    return slots[order[:part.n_sel]]


def select_topk(scores, T: int, P: int, B: int, R: int) -> np.ndarray:
    """Kept slots (ascending) for one head under the top-n rule."""
    part = partition(T, P, B, R)
    if not part.compress:
        return np.arange(part.T, dtype=np.int32)
    s = canonical_scores(np.asarray(scores)[:part.T])
    return _assemble(part, _top_by_rank(s, part))


def random_uniforms(pos, layer: int, head: int, seq: int, event: int, seed: int) -> np.ndarray:
    """u_j = word (p_j mod 4) of Philox4x32-10(ctr=(p_j div 4, layer<<16|head, seq, event),
    key=seed) / 2^32: each block of the counter-based generator gives the four uniforms of four
    consecutive positions, a distinct word for every distinct position."""
    p = np.asarray(pos, dtype=np.int64).astype(np.uint64) & np.uint64(0xFFFFFFFF)
    n = p.size
    c1 = np.full(n, ((int(layer) << 16) | int(head)) & 0xFFFFFFFF, np.uint64)
    c2 = np.full(n, int(seq) & 0xFFFFFFFF, np.uint64)
    c3 = np.full(n, int(event) & 0xFFFFFFFF, np.uint64)
    k0 = np.full(n, int(seed) & 0xFFFFFFFF, np.uint64)
    k1 = np.full(n, (int(seed) >> 32) & 0xFFFFFFFF, np.uint64)
    words = np.stack(philox4x32_10_np(p >> np.uint64(2), c1, c2, c3, k0, k1))   # (4, n)
    u = words[(p & np.uint64(3)).astype(np.int64), np.arange(n)]
    return u.astype(np.float64) / 4294967296.0


def select_random(T: int, P: int, B: int, R: int, pos: Optional[np.ndarray],
                  seed: int, event: int, layer: int, head: int, seq: int) -> np.ndarray:
    """Kept slots (ascending) for one head under Random Attention's rule."""
    part = partition(T, P, B, R)
    if not part.compress:
        return np.arange(part.T, dtype=np.int32)
    p_all = np.arange(part.T, dtype=np.int64) if pos is None else np.asarray(pos, np.int64)[:part.T]
    u = np.full(part.T, -np.inf)
    u[part.e_lo:part.e_hi] = random_uniforms(p_all[part.e_lo:part.e_hi], layer, head, seq, event, seed)
    return _assemble(part, _top_by_rank(u, part))


def select_recent(T: int, P: int, B: int, R: int) -> np.ndarray:
    """Kept slots (ascending) under recency+prompt: the prompt plus the latest slots."""
    part = partition(T, P, B, R)
    if not part.compress:
        return np.arange(part.T, dtype=np.int32)
    latest = np.arange(part.e_hi - part.n_sel, part.e_hi)      # the n_sel latest evictable slots
    return _assemble(part, latest)


def select_random_shared(T: int, P: int, B: int, R: int, pos: Optional[np.ndarray],
                         seed: int, event: int, seq: int) -> np.ndarray:
    """The shared-draw control: one keep-set for every head, drawn as layer 0 / KV head 0's."""
    return select_random(T, P, B, R, pos, seed, event, 0, 0, seq)


def select_union(head_scores, combined, T: int, P: int, B: int, R: int, k: Optional[int] = None) -> np.ndarray:
    """Kept slots (ascending) under union-based selection over the G query heads of a KV head.

    1. every query head g takes its own top-k evictable slots by head_scores[g];
    2. the union of those sets is formed;
    3. the n_sel slots of the union ranked first by the combined score are kept;
    4. if the union holds fewer than n_sel slots, the rest of the evictable range
       tops it up in combined-score order.
    """
    part = partition(T, P, B, R)
    if not part.compress:
        return np.arange(part.T, dtype=np.int32)
    hs = np.atleast_2d(np.asarray(head_scores))
    G = hs.shape[0]
    if k is None:
        k = -(-part.n_sel // G)
    union = set()
    slots = np.arange(part.e_lo, part.e_hi, dtype=np.int64)
    for g in range(G):
        v = canonical_scores(hs[g][:part.T])[part.e_lo:part.e_hi]
        order = np.lexsort((slots, -v))
        union.update(int(x) for x in slots[order[:k]])
    c = canonical_scores(np.asarray(combined)[:part.T])[part.e_lo:part.e_hi]
    in_u = np.array([int(x) in union for x in slots], dtype=bool)   # bool also when the range is empty
    order = np.lexsort((slots, -c, ~in_u))   # union first, then combined score desc, then slot asc
    return _assemble(part, slots[order[:part.n_sel]])

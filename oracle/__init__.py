"""CPU oracle for the KV-eviction hot path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 NumPy statement of what the hot path computes, written
from the pages' definitions:

  * ``score_literal``  -- the averaged RoPE query-centre/key logit, computed
    literally: rotate both vectors, take the real dot product, average over
    the future offsets (TriAttention summary, section 3.4: "RoPE in complex
    form", "The attention dot product in complex form", "Handling Multiple
    Future Positions").
  * ``score_series`` / ``score_folded`` -- the same number through the
    trigonometric series and through the angle-addition expansion; used as
    cross-checks of each other and of the literal form.
  * ``norm_term`` / ``score_full`` -- the norm-based term S_norm weighted by
    one minus the mean resultant length, and S_trig + S_norm (TriAttention
    summary 3.4 "The Norm-Based Term", "Adaptive Weighting").
  * ``score_gqa`` -- per-query-head scores, z-normalised per query head over
    the cached keys, maximum over the query heads of a KV head (summary 3.4,
    GQA handling).
  * ``score_gqa_rotated`` -- the same grouped-query rule over keys stored
    after RoPE.
  * ``score_rotated`` -- the same score for keys stored after RoPE
    (interleaved or half-split pairing), as serving engines keep them.
  * ``partition`` / ``select_topk`` -- prompt and recent-window pinning and
    exact top-n selection (TriAttention summary 3.4 "KV Cache Pruning
    Procedure"; Random Attention section 2 Eq. 2 and section 3 rule 1).
  * ``philox4x32_10`` / ``select_random`` -- per-head uniform random eviction
    (Random Attention section 3, Eq. 3 and Algorithm 1) with a Philox4x32-10
    counter-based generator written from its published description
    (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2,
    3", SC'11).
  * ``compact`` -- the chronological gather of kept rows (Random Attention,
    Appendix F "Engine details"); ``compact_holes`` -- the in-place variant
    that moves only kept rows beyond the new length into evicted slots.
  * ``select_recent`` / ``select_random_shared`` / ``select_union`` -- the
    recency+prompt and shared-draw controls (Random Attention sections 4.1,
    5.2-5.3) and union-based selection (TriAttention blog, eviction step).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product package
(``eviction_long_reasoning_amd``) never imports it, and this package imports
nothing from the product: the two share only the seeded input generators in
``workloads``.

Every function is pinned by ``-m "not gpu"`` tests against closed forms,
invariants, brute force and an independent library Philox; none is marked
"parity unpinned".
"""
from .rope import band_frequencies, band_slices, rope_rotate
from .score import (score_literal, score_series, score_folded, fold_coefficients, norm_term, score_full, score_rotated,
                    score_gqa, score_gqa_rotated, zscore)
from .policy import (Partition, partition, canonical_scores, select_topk, select_random, random_uniforms,
                     select_recent, select_random_shared, select_union)
from .philox import philox4x32_10, philox4x32_10_np, PHILOX_M, PHILOX_W
from .compact import compact, compact_holes

__all__ = [
    "band_frequencies", "band_slices", "rope_rotate",
    "score_literal", "score_series", "score_folded", "fold_coefficients", "norm_term", "score_full", "score_rotated", "score_gqa", "score_gqa_rotated", "zscore",
    "Partition", "partition", "canonical_scores", "select_topk", "select_random", "random_uniforms",
    "select_recent", "select_random_shared", "select_union",
    "philox4x32_10", "philox4x32_10_np", "PHILOX_M", "PHILOX_W",
    "compact", "compact_holes",
]

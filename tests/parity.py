"""Parity rules between the HIP path and the oracle (test helpers).

Scores: fp32 results must satisfy |s - s_ref| <= 1e-4 * max(|s_ref|, rms_h),
where rms_h is the RMS of the oracle's scores over the head's T slots. (A
pure relative error is undefined where the signed sum of cosines crosses
zero, so the head's RMS floors the scale.)

Selection on the GPU's own scores is compared bit-exactly by feeding both
sides identical generated fp32 scores. End to end, the kept sets must have
equal size and may differ only in evictable slots whose oracle score lies
within the same tolerance of the head's selection threshold (the n_sel-th
largest oracle score of the evictable range).

Union-based selection compounds G + 1 rankings. End to end it must (1) give
exactly the oracle's union rule applied to the GPU's own scores, and (2) differ
from the oracle's rule on the oracle's scores only at evictable slots that sit
within tolerance of one of the rule's thresholds: a query head's k-th head
score (the raw-score rule above), or the final combined threshold -- the lowest
combined score the combined ranking chose -- of either run (the z rule). The
second run's threshold covers the slot at the boundary that a changed union
member displaces.

Compaction and the random selector are bit-exact.
"""
from __future__ import annotations

import sys

import numpy as np

from oracle import canonical_scores, partition, select_union
from workloads import bf16_to_f32

SCORE_RTOL = 1e-4


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def keys_f64(K, dtype: str) -> np.ndarray:
    """Exact fp64 image of stored keys (fp32 array or uint16 bf16 bits)."""
    if dtype == "bf16":
        return bf16_to_f32(np.asarray(K)).astype(np.float64)
    return np.asarray(K, dtype=np.float32).astype(np.float64)


def score_errors(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per-slot error in units of the tolerance scale (pass iff every value <= 1e-4)."""
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return np.zeros(0)
    rms = np.sqrt(np.mean(ref ** 2))
    scale = np.maximum(np.abs(ref), rms)
    scale = np.where(scale > 0, scale, 1.0)
    return np.abs(np.asarray(gpu, np.float64) - ref) / scale


def assert_scores(gpu, ref, what=""):
    err = score_errors(gpu, ref)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= SCORE_RTOL, f"{what}: worst scaled score error {worst:.3e} > {SCORE_RTOL}"
    return worst


Z_TOL = 1e-4


def assert_z(gpu, ref, what=""):
    """Normalised (z) scores: |z - z_ref| <= 1e-4 * max(|z_ref|, 1).

    A z-score is a dimensionless O(1) quantity, so unit scale floors the
    relative rule the same way the head RMS floors it for raw scores.
    """
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    err = np.abs(np.asarray(gpu, np.float64) - ref) / np.maximum(np.abs(ref), 1.0)
    worst = float(err.max())
    assert worst <= Z_TOL, f"{what}: worst scaled z error {worst:.3e} > {Z_TOL}"
    return worst


def assert_selection_near_threshold(gpu_kept, ref_kept, ref_scores, T, P, B, R, what=""):
    """End-to-end kept-set rule: equal size; differences only at near-threshold evictable slots."""
    g = set(int(x) for x in gpu_kept)
    r = set(int(x) for x in ref_kept)
    assert len(g) == len(r) == len(gpu_kept), f"{what}: kept sizes {len(g)} vs {len(r)}"
    diff = g ^ r
    if not diff:
        return 0
    p = partition(T, P, B, R)
    s = canonical_scores(np.asarray(ref_scores)[:T])
    ev = s[p.e_lo:p.e_hi]
    thr = np.sort(ev)[::-1][p.n_sel - 1]
    rms = np.sqrt(np.mean(s[np.isfinite(s)] ** 2))
    tol = SCORE_RTOL * max(abs(thr), rms)
    for j in diff:
        assert p.e_lo <= j < p.e_hi, f"{what}: pinned slot {j} differs"
        assert abs(s[j] - thr) <= tol, f"{what}: slot {j} score {s[j]} not within {tol} of threshold {thr}"
    return len(diff)


def kept_rows(kept_row: np.ndarray, n: int) -> np.ndarray:
    return np.asarray(kept_row[:n], dtype=np.int64)


def _union_parts(head, comb, T, P, B, R):
    """For one run of the union rule: the union of the per-head top-k sets, the per-head k-th
    values, and the kept set it gives."""
    p = partition(T, P, B, R)
    hs = np.atleast_2d(np.asarray(head, np.float64))
    G = hs.shape[0]
    k = -(-p.n_sel // G)
    slots = np.arange(p.e_lo, p.e_hi, dtype=np.int64)
    union, kth = set(), []
    for g in range(G):
        v = canonical_scores(hs[g][:T])[p.e_lo:p.e_hi]
        order = np.lexsort((slots, -v))
        union.update(int(x) for x in slots[order[:k]])
        kth.append(v[order[min(k, v.size) - 1]] if v.size else np.nan)
    kept = select_union(hs, comb, T, P, B, R)
    return p, union, np.asarray(kth), kept


def _combined_threshold(p, union, kept, comb):
    """Lowest combined score among the slots the combined ranking chose (None if it chose none)."""
    chosen = [int(j) for j in kept if p.e_lo <= j < p.e_hi]
    if len(union) < p.n_sel:                       # short union: the top-up came from the combined ranking
        chosen = [j for j in chosen if j not in union]
    if not chosen:
        return None
    c = canonical_scores(np.asarray(comb)[:p.T])
    return float(np.min(c[chosen]))


def assert_union_near_thresholds(gpu_kept, gpu_head, gpu_comb, ref_head, ref_comb, T, P, B, R, what=""):
    """The end-to-end union rule of the module docstring; returns the number of differing slots."""
    g = np.asarray(gpu_kept, np.int64)
    exact = select_union(np.asarray(gpu_head, np.float64), np.asarray(gpu_comb, np.float64), T, P, B, R)
    assert np.array_equal(g, exact), f"{what}: the GPU union differs from the rule on the GPU's own scores"
    p, u_ref, kth_ref, ref_kept = _union_parts(ref_head, ref_comb, T, P, B, R)
    assert g.size == ref_kept.size, f"{what}: kept sizes {g.size} vs {ref_kept.size}"
    diff = set(g.tolist()) ^ set(ref_kept.tolist())
    if not diff:
        return 0
    pg, u_gpu, _, _ = _union_parts(gpu_head, gpu_comb, T, P, B, R)
    thr_ref = _combined_threshold(p, u_ref, ref_kept, ref_comb)
    thr_gpu = _combined_threshold(pg, u_gpu, g, gpu_comb)
    hs = np.atleast_2d(np.asarray(ref_head, np.float64))
    c_ref = canonical_scores(np.asarray(ref_comb)[:T])
    c_gpu = canonical_scores(np.asarray(gpu_comb)[:T])
    for j in diff:
        assert p.e_lo <= j < p.e_hi, f"{what}: pinned slot {j} differs"
        near = False
        for gq in range(hs.shape[0]):
            s = canonical_scores(hs[gq][:T])
            rms = np.sqrt(np.mean(s[np.isfinite(s)] ** 2)) if np.isfinite(s).any() else 0.0
            if abs(s[j] - kth_ref[gq]) <= SCORE_RTOL * max(abs(kth_ref[gq]), rms):
                near = True
                break
        for thr, c in ((thr_ref, c_ref), (thr_gpu, c_gpu)):
            if not near and thr is not None and abs(c[j] - thr) <= Z_TOL * max(abs(thr), 1.0):
                near = True
        assert near, f"{what}: slot {j} is near no threshold of the union rule"
    return len(diff)

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

Compaction and the random selector are bit-exact.
"""
from __future__ import annotations

import sys

import numpy as np

from oracle import canonical_scores, partition
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

"""Key scores from the query centre -- oracle (test infrastructure only).

What is computed (one KV head): for each cached key k_j at position p_j and
the current position t,

    S_j = (1/|D|) * sum_{delta in D} < RoPE(q_bar, t + delta), RoPE(k_j, p_j) >

where <.,.> is the real dot product. This is the trigonometric-series term
S_trig of the TriAttention summary (section 3.4 "TriAttention Key Importance
Scoring: The Trigonometric Series Term", with the query replaced by its
centre and the actual key kept) averaged over the future offsets D as in
"Handling Multiple Future Positions" (the future query sits at the key's age
plus delta; age + delta = t + delta - p_j). No 1/sqrt(d) factor appears in
S_trig, so none is applied. The centre q_bar is supplied per KV head.

Three independent evaluations are provided:
  * ``score_literal`` -- rotate both vectors, dot, average (the definition);
  * ``score_series``  -- sum_f |q_f||k_f| cos(omega_f Delta + phi_f), the
    form of the summary's "attention dot product in complex form" with
    phi_f = arg q_f - arg k_f;
  * ``score_folded``  -- angle addition moves the offset average into one
    complex coefficient per band, A_f = mean_delta exp(i omega_f delta), so
    S_j = sum_f Re(q_f A_f conj(k_f) exp(i omega_f (t - p_j))). The
    TriAttention blog's implementation walkthrough computes the same
    Re(q_centre * conj(k) * exp(i phase)) product per band.

The oracle's reference value is ``score_literal``.

The full TriAttention score adds the norm-based term of the same section
("The Norm-Based Term", "Adaptive Weighting via Q/K Concentration"):

    S_norm(k) = sum_f (1 - R_f) * E[|q_f|] * |k_f|,   R_f = |q_bar_f| / E[|q_f|]

which does not depend on the distance, so the offset-averaged full score is
``score_full = score_literal + norm_term``.

Grouped-query attention (summary 3.4 "KV Cache Pruning Procedure", GQA):
each of the G query heads sharing a KV head has its own centre; its scores
are z-normalised over the head's cached keys and the final score is the
maximum over the G query heads (``score_gqa``).

Keys stored after RoPE (the TriAttention blog's implementation walkthrough:
the serving engine keeps rotated keys) are scored by ``score_rotated``: the
same average, with the key already rotated, so no key position is needed.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

from .rope import band_frequencies, band_slices, rope_rotate


def _as_inputs(K, pos, qbar):
    K = np.asarray(K, dtype=np.float64)
    if K.ndim != 2 or K.shape[1] % 2:
        raise ValueError("K must be (T, d) with even d")
    T = K.shape[0]
    pos = np.arange(T, dtype=np.int64) if pos is None else np.asarray(pos, dtype=np.int64)
    q = np.asarray(qbar, dtype=np.float64)
    if pos.shape != (T,) or q.shape != (K.shape[1],):
        raise ValueError("shape mismatch")
    return K, pos, q


def score_literal(K, pos, qbar, t: int, theta: float, deltas: Sequence[int]) -> np.ndarray:
    """Mean over delta of the real dot product of RoPE(q_bar, t+delta) and RoPE(k_j, p_j)."""
    K, pos, q = _as_inputs(K, pos, qbar)
    if len(deltas) == 0:
        raise ValueError("empty offset set")
    k_rot = rope_rotate(K, pos, theta)                      # (T, d), independent of delta
    acc = np.zeros(K.shape[0], dtype=np.float64)
    for delta in deltas:
        q_rot = rope_rotate(q, int(t) + int(delta), theta)  # (d,)
        acc += k_rot @ q_rot
    return acc / len(deltas)


def score_series(K, pos, qbar, t: int, theta: float, deltas: Sequence[int]) -> np.ndarray:
    """Mean over delta of sum_f |q_f| |k_f| cos(omega_f (t + delta - p_j) + arg q_f - arg k_f)."""
    K, pos, q = _as_inputs(K, pos, qbar)
    omega = band_frequencies(K.shape[1], theta)
    qc = q[0::2] + 1j * q[1::2]
    kc = K[:, 0::2] + 1j * K[:, 1::2]
    amp = np.abs(qc)[None, :] * np.abs(kc)                  # (T, F)
    phi = np.angle(qc)[None, :] - np.angle(kc)              # (T, F)
    acc = np.zeros(K.shape[0], dtype=np.float64)
    for delta in deltas:
        dist = (int(t) + int(delta) - pos).astype(np.float64)
        acc += np.sum(amp * np.cos(omega[None, :] * dist[:, None] + phi), axis=1)
    return acc / len(deltas)


def fold_coefficients(d: int, theta: float, deltas: Sequence[int]) -> np.ndarray:
    """A_f = (1/|D|) sum_{delta in D} exp(i omega_f delta), complex128 (F,)."""
    omega = band_frequencies(d, theta)
    dl = np.asarray(list(deltas), dtype=np.float64)
    return np.exp(1j * omega[None, :] * dl[:, None]).mean(axis=0)


def score_folded(K, pos, qbar, t: int, theta: float, deltas: Sequence[int]) -> np.ndarray:
    """sum_f Re(q_f A_f conj(k_f) exp(i omega_f (t - p_j))) -- the angle-addition form."""
    K, pos, q = _as_inputs(K, pos, qbar)
    d = K.shape[1]
    omega = band_frequencies(d, theta)
    u = (q[0::2] + 1j * q[1::2]) * fold_coefficients(d, theta, deltas)
    kc = K[:, 0::2] + 1j * K[:, 1::2]
    age = (int(t) - pos).astype(np.float64)
    rot = np.exp(1j * omega[None, :] * age[:, None])
    return np.real(u[None, :] * np.conj(kc) * rot).sum(axis=1)


def norm_term(K, qbar, qabs) -> np.ndarray:
    """S_norm(k_j) = sum_f (1 - R_f) E|q_f| |k_f| with R_f = |q_bar_f| / E|q_f| (R_f := 1 where E|q_f| = 0)."""
    K = np.asarray(K, dtype=np.float64)
    q = np.asarray(qbar, dtype=np.float64)
    qa = np.asarray(qabs, dtype=np.float64)
    F = K.shape[1] // 2
    if q.shape != (2 * F,) or qa.shape != (F,):
        raise ValueError("shape mismatch")
    centre = np.abs(q[0::2] + 1j * q[1::2])
    with np.errstate(divide="ignore", invalid="ignore"):
        R = np.where(qa > 0, centre / np.where(qa > 0, qa, 1.0), 1.0)
    weight = (1.0 - R) * qa
    k_abs = np.abs(K[:, 0::2] + 1j * K[:, 1::2])
    return k_abs @ weight


def score_full(K, pos, qbar, qabs, t: int, theta: float, deltas: Sequence[int]) -> np.ndarray:
    """Offset-averaged S_trig plus S_norm (the full TriAttention score before GQA aggregation)."""
    return score_literal(K, pos, qbar, t, theta, deltas) + norm_term(K, qbar, qabs)


def score_rotated(K_rot, qbar, t: int, theta: float, deltas: Sequence[int], style: str = "interleaved",
                  qabs=None) -> np.ndarray:
    """Mean over delta of <RoPE(q_bar, t+delta), k_rot_j> for keys stored after RoPE.

    ``style`` is the layout of both q_bar and the stored keys. With ``qabs`` the norm term
    sum_f (1 - R_f) E|q_f| |k_f| is added (rotation leaves |k_f| unchanged).
    """
    K = np.asarray(K_rot, dtype=np.float64)
    q = np.asarray(qbar, dtype=np.float64)
    if K.ndim != 2 or q.shape != (K.shape[1],):
        raise ValueError("shape mismatch")
    acc = np.zeros(K.shape[0], dtype=np.float64)
    for delta in deltas:
        acc += K @ rope_rotate(q, int(t) + int(delta), theta, style)
    out = acc / len(deltas)
    if qabs is not None:
        re, im = band_slices(K.shape[1], style)
        qa = np.asarray(qabs, dtype=np.float64)
        centre = np.hypot(q[re], q[im])
        with np.errstate(divide="ignore", invalid="ignore"):
            R = np.where(qa > 0, centre / np.where(qa > 0, qa, 1.0), 1.0)
        out = out + np.hypot(K[:, re], K[:, im]) @ ((1.0 - R) * qa)
    return out


def zscore(s) -> np.ndarray:
    """(s - mean) / std over all entries, population std; all zeros when the std is 0."""
    s = np.asarray(s, dtype=np.float64)
    if s.size == 0:
        return s.copy()
    mu = s.mean()
    sd = np.sqrt(np.mean((s - mu) ** 2))
    return np.zeros_like(s) if sd == 0 else (s - mu) / sd


def score_gqa(K, pos, qbar_g, t: int, theta: float, deltas: Sequence[int], qabs_g=None):
    """Per-query-head scores, z-normalised per query head over the T cached keys, max over heads.

    ``qbar_g`` is (G, d) and ``qabs_g`` (G, d/2) or None. Returns (final (T,), per_head (G, T)).
    """
    qg = np.asarray(qbar_g, dtype=np.float64)
    per = []
    for g in range(qg.shape[0]):
        if qabs_g is None:
            per.append(score_literal(K, pos, qg[g], t, theta, deltas))
        else:
            per.append(score_full(K, pos, qg[g], np.asarray(qabs_g)[g], t, theta, deltas))
    per = np.stack(per)
    z = np.stack([zscore(row) for row in per])
    return z.max(axis=0), per


def score_gqa_rotated(K_rot, qbar_g, t: int, theta: float, deltas: Sequence[int], style: str = "interleaved",
                      qabs_g=None):
    """The grouped-query rule (``score_gqa``) for keys stored after RoPE: each query head scores the
    rotated keys with ``score_rotated`` (same pairing for keys and centres), z per head, max.

    Returns (final (T,), per_head (G, T)).
    """
    qg = np.asarray(qbar_g, dtype=np.float64)
    per = np.stack([score_rotated(K_rot, qg[g], t, theta, deltas, style,
                                  None if qabs_g is None else np.asarray(qabs_g)[g]) for g in range(qg.shape[0])])
    z = np.stack([zscore(row) for row in per])
    return z.max(axis=0), per

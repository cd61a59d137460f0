"""RoPE in complex form -- oracle (test infrastructure only).

TriAttention summary, section 3.4 "RoPE in complex form": a d-dimensional
vector is split into d/2 two-dimensional frequency bands; band f pairs the
interleaved coordinates x[2f] and x[2f+1] as the complex number
x_f = x[2f] + i x[2f+1], and RoPE at position p multiplies it by
exp(i omega_f p) with omega_f = theta^(-2f/d).
"""
from __future__ import annotations

import numpy as np


def band_frequencies(d: int, theta: float) -> np.ndarray:
    """omega_f = theta^(-2f/d) for f = 0 .. d/2-1, in fp64."""
    if d % 2:
        raise ValueError("head_dim must be even")
    f = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * f / d)


def band_slices(d: int, style: str = "interleaved"):
    """Where band f's real and imaginary parts sit: interleaved (2f, 2f+1) or half-split (f, f+d/2)."""
    if style == "interleaved":
        return slice(0, d, 2), slice(1, d, 2)
    if style == "half":
        return slice(0, d // 2), slice(d // 2, d)
    raise ValueError(f"unknown RoPE style {style!r}")


def rope_rotate(x: np.ndarray, p, theta: float, style: str = "interleaved") -> np.ndarray:
    """RoPE(x, p): rotate each band of x (last axis) by omega_f * p.

    ``x`` has shape (..., d); ``p`` broadcasts against x.shape[:-1].
    The 2-D rotation of (a, b) by angle phi is (a cos phi - b sin phi,
    a sin phi + b cos phi), i.e. multiplication of a + ib by exp(i phi).
    ``style`` says which coordinates form band f: "interleaved" pairs
    x[2f], x[2f+1] (the summary's complex form); "half" pairs x[f], x[f+d/2]
    (the rotate-half layout that some models store).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    omega = band_frequencies(d, theta)
    ang = np.asarray(p, dtype=np.float64)[..., None] * omega
    c, s = np.cos(ang), np.sin(ang)
    re, im = band_slices(d, style)
    a, b = x[..., re], x[..., im]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (d,)), dtype=np.float64)
    out[..., re] = a * c - b * s
    out[..., im] = a * s + b * c
    return out

"""Philox4x32-10 -- oracle (test infrastructure only).

Written from the generator's published description (Salmon, Moraes, Dror,
Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11): a 128-bit
counter (c0, c1, c2, c3) and a 64-bit key (k0, k1) go through 10 rounds.
Each round multiplies c0 and c2 by the two round multipliers into 64-bit
products and re-forms the counter as

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0));

between rounds the key is advanced by the two Weyl constants (the golden
ratio and sqrt(3)-1 scaled to 32 bits). Two implementations: arbitrary
precision Python integers, and a vectorised NumPy one on uint64 lanes (a
32x32 product is exact in 64 bits).
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

PHILOX_M = (0xD2511F53, 0xCD9E8D57)   # round multipliers
PHILOX_W = (0x9E3779B9, 0xBB67AE85)   # Weyl key increments
_MASK = 0xFFFFFFFF


def philox4x32_10(ctr: Sequence[int], key: Sequence[int]) -> Tuple[int, int, int, int]:
    """One Philox4x32-10 block: four 32-bit words from counter and key (Python ints)."""
    c0, c1, c2, c3 = (int(x) & _MASK for x in ctr)
    k0, k1 = (int(x) & _MASK for x in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W[0]) & _MASK
            k1 = (k1 + PHILOX_W[1]) & _MASK
        p0 = PHILOX_M[0] * c0
        p1 = PHILOX_M[1] * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0, p1 & _MASK, (p0 >> 32) ^ c3 ^ k1, p0 & _MASK)
    return c0, c1, c2, c3


def philox4x32_10_np(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10 over uint64 arrays holding 32-bit values."""
    m = np.uint64(_MASK)
    s32 = np.uint64(32)
    c0, c1, c2, c3, k0, k1 = (np.asarray(x, dtype=np.uint64) & m for x in (c0, c1, c2, c3, k0, k1))
    M0, M1 = np.uint64(PHILOX_M[0]), np.uint64(PHILOX_M[1])
    W0, W1 = np.uint64(PHILOX_W[0]), np.uint64(PHILOX_W[1])
    for rnd in range(10):
        if rnd:
            k0 = (k0 + W0) & m
            k1 = (k1 + W1) & m
        p0 = M0 * c0
        p1 = M1 * c2
        c0, c1, c2, c3 = ((p1 >> s32) ^ c1 ^ k0, p1 & m, (p0 >> s32) ^ c3 ^ k1, p0 & m)
    return c0, c1, c2, c3

"""Pins for the oracle's gather-compaction (CPU only)."""
import numpy as np
import pytest

from oracle import compact
from workloads import random_kept


def test_rows_carry_their_source_index():
    T, d = 50, 6
    K = np.repeat(np.arange(T, dtype=np.float32)[:, None], d, 1)
    V = -K
    kept = random_kept(1, T, 17)
    Ko, Vo, po = compact(K, V, None, kept)
    assert np.all(Ko[:, 0] == kept) and np.all(Vo[:, 3] == -kept.astype(np.float32))
    assert po.tolist() == kept.tolist()


def test_positions_follow_rows_and_identity():
    T, d = 20, 4
    K = np.arange(T * d, dtype=np.float32).reshape(T, d)
    pos = np.arange(T, dtype=np.int32) * 7 + 3
    Ko, Vo, po = compact(K, K, pos, np.arange(T))
    assert np.array_equal(Ko, K) and np.array_equal(po, pos)
    _, _, po = compact(K, K, pos, [2, 5, 19])
    assert po.tolist() == [17, 38, 136]


def test_out_of_range_raises():
    with pytest.raises(IndexError):
        compact(np.zeros((4, 2)), np.zeros((4, 2)), None, [0, 4])

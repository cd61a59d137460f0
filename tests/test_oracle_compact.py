"""Pins for the oracle's gather-compaction (CPU only)."""
import numpy as np
import pytest

from oracle import compact, compact_holes
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


# ---------------------------------------------------------------- in-place hole filling ----
def test_holes_hand_example():
    # kept {0, 2, 3, 7} of 10 slots: the only hole below 4 is slot 1, filled by slot 7
    K = np.arange(10, dtype=np.float32)[:, None] * np.ones((1, 3), np.float32)
    Kc, Vc, pc, moves = compact_holes(K, -K, None, [0, 2, 3, 7])
    assert moves == [(7, 1)]
    assert Kc[:, 0].tolist() == [0, 7, 2, 3] and pc.tolist() == [0, 7, 2, 3]


@pytest.mark.parametrize("seed", range(6))
def test_holes_is_a_permutation_of_the_gather(seed):
    T, d = 300, 4
    r = np.random.default_rng(seed)
    K = r.standard_normal((T, d)).astype(np.float32)
    V = r.standard_normal((T, d)).astype(np.float32)
    pos = np.sort(r.choice(10_000, size=T, replace=False)).astype(np.int32)
    kept = random_kept(seed, T, int(r.integers(1, T)))
    gK, gV, gp = compact(K, V, pos, kept)
    hK, hV, hp, moves = compact_holes(K, V, pos, kept)
    n = len(kept)
    # the same rows, each with its own position, in another order
    assert sorted(map(tuple, np.c_[hp, hK, hV].tolist())) == sorted(map(tuple, np.c_[gp, gK, gV].tolist()))
    # a kept row already below n stays in its slot
    ks = set(int(x) for x in kept)
    for x in range(n):
        if x in ks:
            assert hp[x] == pos[x] and np.array_equal(hK[x], K[x])
    # exactly the kept rows at or beyond n move, each into an evicted slot below n
    assert len(moves) == sum(1 for x in kept if x >= n) == n - sum(1 for x in kept if x < n)
    assert all(src >= n and dst < n and dst not in ks for src, dst in moves)


def test_holes_nothing_moves_when_the_kept_set_is_a_prefix():
    K = np.arange(12, dtype=np.float32)[:, None]
    Kc, _, pc, moves = compact_holes(K, K, None, range(8))
    assert moves == [] and pc.tolist() == list(range(8))

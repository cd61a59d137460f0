"""Property tests of the oracle over random tiny heads (CPU only): the partition arithmetic, the
selectors' structure and ranking rule (stated a second way, with Python's own sort), hole filling
against the gather, and the score's three statements (literal RoPE dot product, series, fold), its
dependence on t - p only, and its post-RoPE form."""
import math

import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import (compact, compact_holes, partition, random_uniforms, rope_rotate, score_folded, score_literal,
                    score_rotated, score_series, select_random, select_recent, select_topk, select_union)

SETTINGS = settings(max_examples=80, deadline=None)

# small shapes around the interesting boundaries: T <= B, P >= B, P + R > B, empty evictable range
shapes = st.tuples(st.integers(0, 48), st.integers(0, 60), st.integers(1, 40), st.integers(0, 16)).map(
    lambda x: (x[0], min(x[1], x[0]), x[2], x[3]))     # (T, P, B, R) with P <= T
# scores from a small pool so that ties, NaN, signed zeros and infinities all occur
score_pool = st.sampled_from([0.0, -0.0, 1.0, -1.0, 0.5, 2.5, -7.0, math.inf, -math.inf, math.nan, 1e-30, 3.0])


def _rank_key(x: float):
    """The ranking rule stated directly: NaN ranks as -inf, -0.0 equals +0.0."""
    if x != x:
        return -math.inf
    return 0.0 if x == 0.0 else x


def _check_structure(kept, T, P, B, R):
    p = partition(T, P, B, R)
    kept = [int(x) for x in kept]
    assert kept == sorted(set(kept)), "ascending, no repeats"
    assert all(0 <= j < T for j in kept)
    if T <= B:
        assert kept == list(range(T))
        return p, kept
    assert len(kept) == max(B, P) == p.n_kept
    assert set(range(P)) <= set(kept), "the prompt is kept"
    assert set(range(T - p.R, T)) <= set(kept), "the recent window is kept"
    assert p.R == min(R, max(0, B - P), T - P)
    assert p.n_sel == max(0, B - P - p.R) and p.e_lo == P and p.e_hi == T - p.R
    return p, kept


@SETTINGS
@given(shapes)
def test_partition_arithmetic(shape):
    T, P, B, R = shape
    p = partition(T, P, B, R)
    if T <= B:
        assert not p.compress and p.n_kept == T
        return
    assert p.compress
    assert 0 <= p.e_lo <= p.e_hi <= T
    assert p.n_sel <= p.e_hi - p.e_lo
    # prompt + recent window + selected = kept whenever the prompt fits the budget
    if P <= B:
        assert P + p.R + p.n_sel == B == p.n_kept
    else:
        assert p.R == 0 and p.n_sel == 0 and p.n_kept == P


@SETTINGS
@given(shapes, st.lists(score_pool, min_size=48, max_size=48))
def test_topk_keeps_the_best_ranked_candidates(shape, pool):
    T, P, B, R = shape
    scores = np.array(pool[:T], dtype=np.float32)
    kept = select_topk(scores, T, P, B, R)
    p, kept = _check_structure(kept, T, P, B, R)
    if T <= B:
        return
    ranked = sorted(range(p.e_lo, p.e_hi), key=lambda j: (-_rank_key(float(scores[j])), j))
    want = set(ranked[:p.n_sel])
    assert set(kept) - set(range(P)) - set(range(T - p.R, T)) == want


@SETTINGS
@given(shapes, st.integers(0, 2 ** 64 - 1), st.integers(0, 1000), st.integers(0, 7), st.integers(0, 7),
       st.integers(0, 7))
def test_random_keeps_the_largest_uniforms(shape, seed, event, layer, head, seq):
    T, P, B, R = shape
    kept = select_random(T, P, B, R, None, seed, event, layer, head, seq)
    p, kept = _check_structure(kept, T, P, B, R)
    if T <= B:
        return
    u = random_uniforms(np.arange(p.e_lo, p.e_hi), layer, head, seq, event, seed)
    assert np.all((u >= 0.0) & (u < 1.0))
    ranked = sorted(range(p.e_lo, p.e_hi), key=lambda j: (-u[j - p.e_lo], j))
    assert set(kept) - set(range(P)) - set(range(T - p.R, T)) == set(ranked[:p.n_sel])


@SETTINGS
@given(shapes)
def test_recent_keeps_the_latest_candidates(shape):
    T, P, B, R = shape
    p, kept = _check_structure(select_recent(T, P, B, R), T, P, B, R)
    if T > B:
        assert set(kept) - set(range(P)) - set(range(T - p.R, T)) == set(range(p.e_hi - p.n_sel, p.e_hi))


@SETTINGS
@given(shapes, st.integers(1, 4), st.lists(score_pool, min_size=4 * 48, max_size=4 * 48),
       st.lists(score_pool, min_size=48, max_size=48))
def test_union_structure_and_k_equal_n_sel(shape, G, pool, comb):
    T, P, B, R = shape
    hs = np.array(pool[:G * T], dtype=np.float32).reshape(G, T) if T else np.zeros((G, 0), np.float32)
    combined = np.array(comb[:T], dtype=np.float32)
    _check_structure(select_union(hs, combined, T, P, B, R), T, P, B, R)
    # with k = n_sel every head's own top set alone already fills the budget: the union keeps the
    # n_sel slots of the union ranked first by the combined score
    p = partition(T, P, B, R)
    if T > B and p.n_sel > 0:
        kept = select_union(hs, combined, T, P, B, R, k=p.n_sel)
        heads = set()
        for g in range(G):
            heads |= set(sorted(range(p.e_lo, p.e_hi), key=lambda j: (-_rank_key(float(hs[g, j])), j))[:p.n_sel])
        ranked = sorted(heads, key=lambda j: (-_rank_key(float(combined[j])), j))
        assert set(kept) - set(range(P)) - set(range(T - p.R, T)) == set(ranked[:p.n_sel])


@SETTINGS
@given(shapes, st.integers(0, 2 ** 32 - 1))
def test_hole_filling_is_a_permutation_of_the_gather(shape, seed):
    T, P, B, R = shape
    kept = select_random(T, P, B, R, None, seed, 1, 0, 0, 0)
    n = len(kept)
    K = np.arange(T * 2, dtype=np.float32).reshape(T, 2)        # every row names its slot
    V = -K
    pos = (np.arange(T) * 3 + 7).astype(np.int32)
    gk, gv, gp = compact(K, V, pos, kept)
    hk, hv, hp, moves = compact_holes(K, V, pos, kept)
    assert hk.shape == gk.shape and hv.shape == gv.shape
    # the same multiset of rows, with positions travelling with their rows
    assert sorted(map(tuple, hk.tolist())) == sorted(map(tuple, gk.tolist()))
    assert np.array_equal(hp, (hk[:, 0] / 2 * 3 + 7).astype(np.int32))
    assert np.array_equal(hv, -hk)
    # kept rows below n stay where they are; every move goes from a slot >= n into one below n
    for j in kept:
        if j < n:
            assert hk[j, 0] == 2 * j
    assert all(src >= n > dst for src, dst in moves)
    assert len(moves) == sum(1 for j in kept if j >= n)


# ---------------------------------------------------------------- scores ----
score_inputs = st.tuples(
    st.sampled_from([2, 4, 6, 8, 16]),                       # head_dim
    st.integers(1, 6),                                       # keys
    st.sampled_from([1e4, 1e6, 500.0]),                      # theta
    st.lists(st.integers(0, 70000), min_size=1, max_size=5),  # offsets
    st.integers(0, 2 ** 31 - 1),                             # value seed
    st.integers(0, 100000),                                  # current position
)


def _draw(d, n, seed, t):
    r = np.random.default_rng(seed)
    K = r.standard_normal((n, d))
    q = r.standard_normal(d)
    pos = r.integers(0, t + 1, n)
    return K, q, pos


@SETTINGS
@given(score_inputs)
def test_series_and_fold_equal_the_literal_score(args):
    d, n, theta, deltas, seed, t = args
    K, q, pos = _draw(d, n, seed, t)
    lit = score_literal(K, pos, q, t, theta, deltas)
    scale = np.linalg.norm(q) * np.linalg.norm(K, axis=1) + 1e-300
    # three statements of one quantity agree to a few ulps of the angles they reduce
    for other in (score_series(K, pos, q, t, theta, deltas), score_folded(K, pos, q, t, theta, deltas)):
        assert np.all(np.abs(other - lit) <= 1e-9 * scale), (other, lit)


@SETTINGS
@given(score_inputs, st.integers(-5000, 5000))
def test_score_depends_on_t_minus_p_only(args, shift):
    d, n, theta, deltas, seed, t = args
    K, q, pos = _draw(d, n, seed, t)
    if t + shift < 0 or np.any(pos + shift < 0):
        return
    a = score_folded(K, pos, q, t, theta, deltas)
    b = score_folded(K, pos + shift, q, t + shift, theta, deltas)
    scale = np.linalg.norm(q) * np.linalg.norm(K, axis=1) + 1e-300
    assert np.all(np.abs(a - b) <= 1e-9 * scale)


@SETTINGS
@given(score_inputs, st.sampled_from(["interleaved", "half"]))
def test_rotated_keys_give_the_pre_rope_score(args, style):
    d, n, theta, deltas, seed, t = args
    K, q, _ = _draw(d, n, seed, t)
    slots = np.arange(n)
    if style == "interleaved":
        ref = score_literal(K, slots, q, t, theta, deltas)
        got = score_rotated(rope_rotate(K, slots, theta, style), q, t, theta, deltas, style)
    else:
        # half-split storage is the interleaved layout under a fixed permutation of coordinates
        perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
        ref = score_literal(K, slots, q, t, theta, deltas)
        got = score_rotated(rope_rotate(K[:, perm], slots, theta, style), q[perm], t, theta, deltas, style)
    scale = np.linalg.norm(q) * np.linalg.norm(K, axis=1) + 1e-300
    assert np.all(np.abs(got - ref) <= 1e-9 * scale)

"""The end-to-end union rule of tests/parity.py, pinned on the CPU: it accepts a kept set that
differs from the oracle's only through near-threshold perturbations (including the boundary slot a
changed union member displaces), and rejects one that differs anywhere else or that the union rule
does not produce from the GPU-side scores."""
import numpy as np
import pytest

import oracle
from parity import assert_union_near_thresholds


def _case(seed, G=4, T=400, P=40, B=120, R=16):
    r = np.random.default_rng(seed)
    head = r.standard_normal((G, T))
    comb = head.max(axis=0)
    return head, comb, T, P, B, R


def test_identical_scores_differ_nowhere():
    head, comb, T, P, B, R = _case(1)
    kept = oracle.select_union(head, comb, T, P, B, R)
    assert assert_union_near_thresholds(kept, head, comb, head, comb, T, P, B, R) == 0


def test_tiny_perturbations_are_accepted():
    # scores within 1e-6 relative of the oracle's: any swap they cause sits at a threshold
    for seed in range(20):
        head, comb, T, P, B, R = _case(seed)
        r = np.random.default_rng(100 + seed)
        gh = head * (1 + 1e-6 * r.standard_normal(head.shape))
        gc = gh.max(axis=0)
        kept = oracle.select_union(gh, gc, T, P, B, R)
        assert_union_near_thresholds(kept, gh, gc, head, comb, T, P, B, R, f"seed {seed}")


def test_a_swap_forced_at_a_head_threshold_is_accepted():
    # the oracle's scores put slot b just below head g's k-th member a; the GPU side, within 1e-7
    # relative, puts it just above: b joins the union instead of a, and the final ranking may
    # displace its boundary slot in turn
    differing = 0
    for seed in range(12):
        head, comb, T, P, B, R = _case(40 + seed)
        p = oracle.partition(T, P, B, R)
        k = -(-p.n_sel // head.shape[0])
        g = seed % head.shape[0]
        v = head[g, p.e_lo:p.e_hi]
        order = np.argsort(-v, kind="stable")
        a, b = p.e_lo + order[k - 1], p.e_lo + order[k]
        head[g, b] = head[g, a] * (1 - 1e-7) if head[g, a] > 0 else head[g, a] * (1 + 1e-7)
        comb = head.max(axis=0)
        gh = head.copy()
        gh[g, b] = head[g, a] * (1 + 1e-7) if head[g, a] > 0 else head[g, a] * (1 - 1e-7)
        gc = gh.max(axis=0)
        kept = oracle.select_union(gh, gc, T, P, B, R)
        differing += assert_union_near_thresholds(kept, gh, gc, head, comb, T, P, B, R, f"seed {seed}")
    assert differing > 0    # some of the forced flips change the kept set


def test_far_difference_is_rejected():
    head, comb, T, P, B, R = _case(3)
    p = oracle.partition(T, P, B, R)
    gh = head.copy()
    j = p.e_lo + int(np.argmin(comb[p.e_lo:p.e_hi]))   # the lowest-scored evictable slot
    gh[:, j] = 50.0                                      # far above every threshold on the GPU side
    gc = gh.max(axis=0)
    kept = oracle.select_union(gh, gc, T, P, B, R)
    assert j in set(kept.tolist())
    with pytest.raises(AssertionError, match="near no threshold"):
        assert_union_near_thresholds(kept, gh, gc, head, comb, T, P, B, R)


def test_kept_set_not_produced_by_the_rule_is_rejected():
    head, comb, T, P, B, R = _case(4)
    kept = oracle.select_union(head, comb, T, P, B, R).copy()
    p = oracle.partition(T, P, B, R)
    sel = [i for i, j in enumerate(kept) if p.e_lo <= j < p.e_hi]
    outside = sorted(set(range(p.e_lo, p.e_hi)) - set(kept.tolist()))
    kept[sel[0]] = outside[0]                            # an off-by-one style slip in the kept list
    kept.sort()
    with pytest.raises(AssertionError, match="own scores"):
        assert_union_near_thresholds(kept, head, comb, head, comb, T, P, B, R)

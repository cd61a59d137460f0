"""Pins for the oracle's pinning, top-n selection and random selection (CPU only)."""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import (canonical_scores, partition, philox4x32_10, random_uniforms, select_random, select_random_shared,
                    select_recent, select_topk, select_union)
from workloads import random_scores, rng

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "partition_cases.json")


def _f32(vals):
    return np.array([float(v) for v in vals], dtype=np.float32)


# --------------------------------------------------------------------------
# hand-worked cases
# --------------------------------------------------------------------------
def test_partition_golden():
    for c in json.load(open(GOLDEN))["partition"]:
        p = partition(c["T"], c["P"], c["B"], c["R"])
        got = dict(e_lo=p.e_lo, e_hi=p.e_hi, n_sel=p.n_sel, n_kept=p.n_kept, compress=p.compress)
        exp = {k: c[k] for k in got}
        assert got == exp, c["name"]


def test_select_golden():
    for c in json.load(open(GOLDEN))["select"]:
        kept = select_topk(_f32(c["scores"]), c["T"], c["P"], c["B"], c["R"])
        assert kept.tolist() == c["kept"], c["name"]


def test_canonical_scores():
    s = canonical_scores(_f32(["nan", "-0.0", "0.0", "inf", "-inf", "1.5"]))
    assert s[0] == -np.inf and np.signbit(s[1]) == False and s[3] == np.inf and s[5] == 1.5


# --------------------------------------------------------------------------
# the characterising invariant and brute force
# --------------------------------------------------------------------------
def _beats(sa, a, sb, b):
    return sa > sb or (sa == sb and a < b)


def _check_kept(kept, scores, T, P, B, R):
    p = partition(T, P, B, R)
    kept = np.asarray(kept)
    assert kept.size == p.n_kept
    assert np.all(np.diff(kept) > 0) and (kept.size == 0 or (kept[0] >= 0 and kept[-1] < T))
    if not p.compress:
        assert kept.tolist() == list(range(T))
        return
    ks = set(kept.tolist())
    pins = set(range(p.P)) | set(range(T - p.R, T))
    assert pins <= ks
    sel = sorted(ks - pins)
    assert len(sel) == p.n_sel and all(p.e_lo <= j < p.e_hi for j in sel)
    s = canonical_scores(scores)
    rest = [j for j in range(p.e_lo, p.e_hi) if j not in ks]
    for a in sel:
        for b in rest:
            assert _beats(s[a], a, s[b], b)


@pytest.mark.parametrize("seed", range(40))
def test_selection_invariant_random(seed):
    r = rng(200, seed)
    T = int(r.integers(0, 80))
    P = int(r.integers(0, 20))
    B = int(r.integers(1, 60))
    R = int(r.integers(0, 12))
    s = random_scores(seed, (max(T, 1),), ties=0.3, specials=bool(seed % 2))[:T]
    _check_kept(select_topk(s, T, P, B, R), s, T, P, B, R)


@pytest.mark.parametrize("seed", range(12))
def test_selection_brute_force(seed):
    # among all n_sel-subsets of the evictable range exactly one dominates the rest under
    # (score desc, slot asc); it must be the oracle's choice
    r = rng(201, seed)
    T, P, R = 14, int(r.integers(0, 3)), int(r.integers(0, 3))
    B = int(r.integers(P + R + 1, T))
    s = random_scores(100 + seed, (T,), ties=0.4, specials=(seed % 3 == 0))
    p = partition(T, P, B, R)
    c = canonical_scores(s)
    E = list(range(p.e_lo, p.e_hi))
    winners = [sub for sub in itertools.combinations(E, p.n_sel)
               if all(_beats(c[a], a, c[b], b) for a in sub for b in E if b not in sub)]
    assert len(winners) == 1
    kept = select_topk(s, T, P, B, R)
    assert sorted(set(kept.tolist()) - set(range(P)) - set(range(T - p.R, T))) == list(winners[0])


def test_budget_counts_every_kept_entry():
    # |kept| = B whenever the prompt fits in the budget (the full-pass workload shape)
    for T, P, B, R in [(32768, 1024, 3072, 128), (32768, 512, 2048, 128), (2176, 2000, 2048, 128)]:
        p = partition(T, P, B, R)
        assert p.n_kept == B and p.P + p.R + p.n_sel == B


# --------------------------------------------------------------------------
# random selection: Random Attention section 3 (Eq. 3, Algorithm 1) and Appendix D
# --------------------------------------------------------------------------
def test_random_kept_structure():
    for seed in range(6):
        T, P, B, R = 300, 40, 100, 16
        kept = select_random(T, P, B, R, None, seed, 3, 1, 2, 5)
        p = partition(T, P, B, R)
        assert kept.size == B and np.all(np.diff(kept) > 0)
        assert set(range(P)) <= set(kept.tolist()) and set(range(T - p.R, T)) <= set(kept.tolist())


def test_random_uniforms_layout():
    # position p draws word p mod 4 of the Philox block with counter (p div 4, layer<<16|head, seq,
    # event) and key (seed mod 2^32, seed >> 32): checked against the scalar generator (itself
    # pinned to an independent implementation), so a wrong counter word, word or key order fails
    layer, head, seq, event, seed = 5, 3, 7, 11, 0x0123456789ABCDEF
    key = (seed & 0xFFFFFFFF, seed >> 32)
    pos = np.array([0, 1, 2, 3, 4, 7, 4097, 4098, 2 ** 31 + 6, 2 ** 32 - 1])
    want = [philox4x32_10((p >> 2, (layer << 16) | head, seq, event), key)[p & 3] / 2 ** 32 for p in pos.tolist()]
    assert np.array_equal(random_uniforms(pos, layer, head, seq, event, seed), np.array(want))
    # the four positions of a block take its four words, so no two positions share a uniform
    quad = random_uniforms(np.arange(8, 12), layer, head, seq, event, seed) * 2 ** 32
    assert quad.tolist() == [float(w) for w in philox4x32_10((2, (layer << 16) | head, seq, event), key)]
    # each argument reaches the draw
    base = random_uniforms(pos, layer, head, seq, event, seed)
    for args in ((layer + 1, head, seq, event, seed), (layer, head + 1, seq, event, seed),
                 (layer, head, seq + 1, event, seed), (layer, head, seq, event + 1, seed),
                 (layer, head, seq, event, seed ^ (1 << 40))):
        assert not np.any(random_uniforms(pos, *args) == base)


def test_random_ranks_follow_uniforms():
    # the selected candidates are exactly those with the n_sel largest uniforms (ties to lower slot)
    T, P, B, R = 120, 10, 50, 8
    p = partition(T, P, B, R)
    u = random_uniforms(np.arange(p.e_lo, p.e_hi), 2, 3, 4, 9, 0xABCDEF0123)
    want = np.arange(p.e_lo, p.e_hi)[np.lexsort((np.arange(u.size), -u))[:p.n_sel]]
    kept = select_random(T, P, B, R, None, 0xABCDEF0123, 9, 2, 3, 4)
    assert sorted(set(kept.tolist()) - set(range(P)) - set(range(T - p.R, T))) == sorted(want.tolist())


def test_random_marginals_uniform():
    # uniform marginals: each evictable slot is kept with probability n_sel/|E|;
    # pairs are kept together with probability n(n-1)/(|E|(|E|-1)).
    T, P, B, R = 40, 4, 14, 4
    p = partition(T, P, B, R)
    nE, n = p.e_hi - p.e_lo, p.n_sel
    trials = 4000
    counts = np.zeros(T)
    pair = 0
    for ev in range(trials):
        kept = select_random(T, P, B, R, None, 0x5EED, ev, 0, 0, 0)
        counts[kept] += 1
        ks = set(kept.tolist())
        pair += (p.e_lo in ks) and (p.e_lo + 1 in ks)
    obs = counts[p.e_lo:p.e_hi]
    expct = trials * n / nE
    chi2 = np.sum((obs - expct) ** 2 / expct)
    # df = nE - 1 = 31; the 0.999 quantile of chi2(31) is about 61.1
    assert chi2 < 61.1, chi2
    assert np.all(counts[:P] == trials) and np.all(counts[T - p.R:] == trials)
    pp = n * (n - 1) / (nE * (nE - 1))
    assert abs(pair / trials - pp) < 4 * math.sqrt(pp * (1 - pp) / trials)


def test_random_heads_and_layers_draw_independently():
    # different heads/layers/sequences must not share a keep-set: expected overlap n^2/|E|
    T, P, B, R = 600, 0, 100, 0
    p = partition(T, P, B, R)
    ov = []
    for ev in range(50):
        a = set(select_random(T, P, B, R, None, 1, ev, 0, 0, 0).tolist())
        for other in [(0, 1, 0), (1, 0, 0), (0, 0, 1)]:
            b = set(select_random(T, P, B, R, None, 1, ev, *other).tolist())
            ov.append(len(a & b))
    assert abs(np.mean(ov) - p.n_sel ** 2 / (p.e_hi - p.e_lo)) < 2.0


def _survival_sim(K, r, lp, events, heads, seed):
    """Periodic random eviction in the page's framework: budget K plus a never-scored buffer r.

    The keep-all budget of the partition is B = K + r with a recent window R = r; r new tokens
    arrive between events. Returns per-age survival estimates.
    """
    surv_num = np.zeros(events + 1)
    surv_den = np.zeros(events + 1)
    for h in range(heads):
        pos = list(range(K + r))                         # cache right after an eviction
        for ev in range(events):
            pos = pos + list(range(pos[-1] + 1, pos[-1] + 1 + r))
            arr = np.array(pos)
            kept = select_random(len(arr), lp, K + r, r, arr, seed, ev, 0, h, 0)
            keep = set(arr[kept].tolist())
            # a candidate that entered the candidate set at event e0 has faced (ev - e0 + 1) draws
            cand = arr[lp:len(arr) - r]
            for p_ in cand.tolist():
                first = 0 if p_ < K + r else (p_ - K - r) // r + 1   # first event as a candidate
                n = ev - first + 1
                if 1 <= n <= events:
                    surv_den[n] += 1
                    surv_num[n] += p_ in keep
            pos = [x for x in pos if x in keep]
    return surv_num, surv_den


def test_random_survival_law():
    # Random Attention Appendix D ("Implicit age bias"): a position survives each eviction with
    # probability (K - l_p)/(K + r - l_p) independently, because the draw is fresh every time.
    K, r, lp = 48, 8, 4
    num, den = _survival_sim(K, r, lp, events=10, heads=40, seed=77)
    q = (K - lp) / (K + r - lp)
    # conditional survival at each draw must be q (not the geometric of a repeated draw)
    ok = den[1:] > 100
    cond = num[1:][ok] / den[1:][ok]
    tol = 4 * np.sqrt(q * (1 - q) / den[1:][ok])
    assert ok.sum() >= 5 and np.all(np.abs(cond - q) < tol), (cond, q)


def test_random_survival_matches_pages_rate():
    # the pages quote about 0.94 per eviction at K=1024, r=64 (small prompt)
    K, r, lp = 1024, 64, 0
    num, den = _survival_sim(K, r, lp, events=3, heads=3, seed=5)
    rate = num[1:].sum() / den[1:].sum()
    assert abs(rate - 0.94) < 0.01 and abs((K - lp) / (K + r - lp) - 0.94) < 0.005


# --------------------------------------------------------------------------
# policy variants: recency+prompt, shared draw, union-based selection
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T,P,B,R", [(10, 2, 6, 1), (100, 0, 30, 8), (100, 40, 30, 8), (50, 5, 50, 3),
                                     (51, 5, 50, 3), (1000, 100, 300, 64), (7, 7, 3, 2)])
def test_recent_is_prompt_plus_latest(T, P, B, R):
    kept = select_recent(T, P, B, R)
    part = partition(T, P, B, R)
    # closed form: the prompt and the n_kept - P latest slots
    want = list(range(min(P, T))) + list(range(T - (part.n_kept - part.P), T))
    assert kept.tolist() == sorted(set(want)) and kept.size == part.n_kept
    # the top-n rule ranking slots by their own index picks the same set
    assert np.array_equal(kept, select_topk(np.arange(T, dtype=np.float64), T, P, B, R))


def test_recent_hand_example():
    # T=10, P=2, B=6, R=1: keep slots 0,1 and the 4 latest
    assert select_recent(10, 2, 6, 1).tolist() == [0, 1, 6, 7, 8, 9]


def test_shared_draw_is_one_keep_set_for_every_head():
    T, P, B, R = 900, 64, 300, 32
    pos = np.arange(T) * 3 + 11
    a = select_random_shared(T, P, B, R, pos, 99, 4, 2)
    assert np.array_equal(a, select_random(T, P, B, R, pos, 99, 4, 0, 0, 2))
    # the per-head rule draws differently for another head; the shared one does not depend on it
    assert not np.array_equal(a, select_random(T, P, B, R, pos, 99, 4, 3, 5, 2))
    assert not np.array_equal(a, select_random_shared(T, P, B, R, pos, 99, 4, 3))


@pytest.mark.parametrize("seed", range(8))
def test_union_with_budget_sized_heads_equals_top_n_of_the_max(seed):
    # with per-head k = n_sel and the combined score max_g s_g, a slot among the n_sel best by
    # its max is among its arg-max head's n_sel best, so the union rule is the top-n rule on
    # the max (continuous scores: no ties)
    r = rng(620, seed)
    G, T, P, B, R = int(r.integers(1, 9)), 600, 40, 200, 16
    hs = r.standard_normal((G, T))
    comb = hs.max(axis=0)
    part = partition(T, P, B, R)
    assert np.array_equal(select_union(hs, comb, T, P, B, R, k=part.n_sel), select_topk(comb, T, P, B, R))


@pytest.mark.parametrize("seed", range(8))
def test_union_keeps_the_whole_union_when_short_and_only_union_when_long(seed):
    r = rng(621, seed)
    G, T, P, B, R = 4, 400, 20, 150, 10
    part = partition(T, P, B, R)
    base = r.standard_normal(T)
    hs = base[None, :] + 0.05 * r.standard_normal((G, T))       # heads agree: the union is short
    comb = r.standard_normal(T)
    for k, short in ((part.n_sel // G, True), (part.n_sel, False)):
        kept = set(select_union(hs, comb, T, P, B, R, k=k).tolist())
        ev = np.arange(part.e_lo, part.e_hi)
        union = set()
        for g in range(G):
            union |= set(ev[np.argsort(-hs[g, part.e_lo:part.e_hi], kind="stable")[:k]].tolist())
        sel = kept - set(range(P)) - set(range(T - part.R, T))
        assert len(sel) == part.n_sel
        if len(union) <= part.n_sel:
            assert union <= sel                       # short union: all of it is kept ...
            rest = sorted(set(ev.tolist()) - union, key=lambda j: (-comb[j], j))
            assert sel - union == set(rest[:part.n_sel - len(union)])   # ... topped up by combined score
        else:
            assert sel <= union                       # long union: the choice stays inside it
            assert sel == set(sorted(union, key=lambda j: (-comb[j], j))[:part.n_sel])
        if short:
            assert len(union) < part.n_sel


def test_union_hand_example():
    # T=8, no prompt or window, B=3 -> n_sel=3; two heads, k=1 each
    hs = np.array([[0, 5, 1, 0, 0, 0, 0, 0],
                   [0, 0, 0, 0, 0, 0, 4, 0]], dtype=np.float64)
    comb = np.array([0, 1, 9, 3, 0, 0, 2, 8], dtype=np.float64)
    # union = {1, 6}; top-up by combined score from the rest: slot 2 (9)
    assert select_union(hs, comb, 8, 0, 3, 0, k=1).tolist() == [1, 2, 6]

"""GPU parity of the selectors' listed path, case by case, against the oracle (bit-exact).

Selections of at most half the candidates first list the keys at or above a cut taken from a
sample (two fixed rounds per thread, R/4 and 3R/4 of its R rounds) and rank and place over that
list; a cut that leaves too few keys or more than the list holds, or a threshold bin too crowded
to rank directly, falls back to the histogram over every key. Selections of more than half (in the
register tiers and the re-reading kernel) list the keys to evict the same way, with the keys
flipped, and place by the ordered scan. Each case below is built so that a given branch runs (the comment says which); every
one must give the oracle's keep-set exactly.
"""
import numpy as np
import pytest
import torch

import eviction_long_reasoning_amd as kv
import oracle
from parity import log
from workloads import rng

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _i32(x) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, np.int32), device=DEV)


def _round_of(t_cap: int) -> np.ndarray:
    """Round index of every slot in the 1024-thread, 32-round tier (wave w holds 64*32 slots from
    w*2048 on, round i the 64 slots from w*2048 + 64*i on)."""
    return (np.arange(t_cap) % 2048) // 64


def _row(pattern: str, r, t_cap: int, T: int, P: int, B: int, R: int) -> np.ndarray:
    """One head's scores; `share` is the fraction of its candidates that are selected, so the tie
    patterns can straddle the threshold."""
    part = oracle.partition(T, P, B, R)
    share = part.n_sel / max(1, part.e_hi - part.e_lo)
    x = r.standard_normal(t_cap).astype(np.float32)
    if pattern == "trend":            # listed keys pile up in the last waves: the slot-order prefix
        x += np.arange(t_cap, dtype=np.float32) * np.float32(4.0 / t_cap)
    elif pattern == "tie-block-over-cap":   # 9000 equal keys above the rest: the count exceeds the list
        x[r.choice(t_cap, 9000, replace=False)] = np.float32(5.0)
    elif pattern == "crowded-low":    # the same from below: 1500 equal keys hold an over-half threshold
        x *= np.float32(0.3)
        idx = r.choice(t_cap, 2500, replace=False)
        x[idx[:1500]] = np.float32(-2.0)
        x[idx[1500:]] = np.float32(-2.5) - np.float32(7.0) * r.random(1000, dtype=np.float32)
    elif pattern == "crowded-bin":    # 1500 equal keys hold the threshold: its list bin is too crowded
        x *= np.float32(0.3)
        idx = r.choice(t_cap, 2500, replace=False)
        x[idx[:1500]] = np.float32(2.0)
        x[idx[1500:]] = np.float32(2.5) + np.float32(7.0) * r.random(1000, dtype=np.float32)
    elif pattern == "ties-straddle":  # a block of equal keys just below the selection's share
        v = np.float32(np.quantile(x[P:T], min(1.0, 1.0 - share + 0.004)))
        x[r.choice(t_cap, max(8, t_cap // 100), replace=False)] = v
    elif pattern == "signed-zeros":   # +0 and -0 tie at the threshold: positives fall just short
        x = -np.abs(x) - np.float32(0.01)
        n_pos = int((share - 0.01) * t_cap)
        idx = r.choice(t_cap, n_pos + min(t_cap // 60, 600), replace=False)
        x[idx[:n_pos]] = -x[idx[:n_pos]]
        zeros = idx[n_pos:]
        x[zeros] = np.where(r.random(zeros.size) < 0.5, np.float32(0.0), np.float32(-0.0))
    elif pattern == "infinities":     # +inf in the list's top bin, -inf and NaN among the rest
        idx = r.choice(t_cap, 900, replace=False)
        x[idx[:300]] = np.inf
        x[idx[300:600]] = -np.inf
        x[idx[600:]] = np.nan
    elif pattern == "sample-high":    # the sampled rounds score far above the rest: the cut is too high
        rounds = _round_of(t_cap)
        x += np.where((rounds == 8) | (rounds == 24), np.float32(100.0), np.float32(0.0))
    elif pattern == "stream-sample-high":   # past the register tiers the sample is 4096 evenly spaced
        n_cand = part.e_hi - part.e_lo      # candidates: raise exactly those
        ns = min(n_cand, 4096)
        x[part.e_lo + (np.arange(ns, dtype=np.int64) * n_cand) // ns] += np.float32(100.0)
    return x


def _scores(pattern: str, seed: int, shape, Ts, Ps, B: int, R: int) -> np.ndarray:
    """[L, S, H, (G,) t_cap] scores, each head drawn by _row with its sequence's partition."""
    r = rng(540, seed)
    t_cap = shape[-1]
    x = np.empty(shape, np.float32)
    for l in range(shape[0]):
        for s in range(shape[1]):
            for idx in np.ndindex(*shape[2:-1]):
                x[(l, s) + idx] = _row(pattern, r, t_cap, Ts[s], Ps[s], B, R)
    return x


# name, t_cap, T per sequence, P per sequence, B, R, pattern
CASES = [
    ("normal-32k", 32768, [32768, 30001], [1024, 17], 3072, 128, "normal"),
    ("trend-32k", 32768, [32768], [1024], 3072, 128, "trend"),
    ("tie-block-over-cap", 32768, [32768], [1024], 3072, 128, "tie-block-over-cap"),
    ("crowded-bin", 32768, [32768], [512], 2500, 100, "crowded-bin"),
    ("ties-straddle", 32768, [32768, 20000], [1024, 0], 3072, 128, "ties-straddle"),
    ("signed-zeros", 32768, [32768], [1000], 3072, 128, "signed-zeros"),
    ("infinities", 32768, [32768], [256], 2048, 64, "infinities"),
    ("sample-high", 32768, [32768], [1024], 3072, 128, "sample-high"),
    # every sampled round lies in the prompt or the recent window: no valid sample, the cut lists
    # every candidate (512 slots of wave 15's rounds 0..7)
    ("empty-sample", 32768, [32768], [30720], 32356, 1536, "normal"),
    # exactly half, and one past half, of the candidates selected: the listed path's gate
    ("half-selected", 8192, [8192], [0], 4064 + 64, 64, "normal"),
    ("over-half-selected", 8192, [8192], [0], 4065 + 64, 64, "normal"),
    # the smaller tiers' lists (256 x 8, 256 x 16, 512 x 16, 1024 x 16)
    ("tier-2048", 2048, [2048, 1999], [100, 0], 400, 16, "ties-straddle"),
    ("tier-4096-over-cap", 4096, [4096], [64], 1700, 16, "normal"),
    ("tier-8192", 8192, [8192, 5000], [256, 3], 1500, 32, "signed-zeros"),
    ("tier-16384", 16384, [16384], [2048], 4000, 128, "trend"),
    # more than half selected: the keys to evict listed with the keys flipped (register tiers)
    ("flip-32k", 32768, [32768, 30001], [1024, 17], 30000, 128, "normal"),
    ("flip-ties-straddle", 32768, [32768, 20000], [1024, 0], 29000, 128, "ties-straddle"),
    ("flip-signed-zeros", 32768, [32768], [1000], 30000, 128, "signed-zeros"),
    ("flip-infinities", 32768, [32768], [256], 31000, 64, "infinities"),
    # the 400th lowest key is -inf (300 -inf and 300 NaN, which ranks as -inf): the ties at -inf
    # keep their 200 lowest slots
    ("flip-at-neg-inf", 32768, [32768], [256], 32368, 64, "infinities"),
    ("flip-crowded-low", 32768, [32768], [512], 30500, 100, "crowded-low"),
    ("flip-trend", 32768, [32768], [1024], 29000, 128, "trend"),
    ("flip-sample-high", 32768, [32768], [1024], 29000, 128, "sample-high"),
    ("flip-tier-2048", 2048, [2048, 1999], [100, 0], 1800, 16, "ties-straddle"),
    ("flip-tier-4096", 4096, [4096, 2176], [64, 300], 3900, 16, "normal"),
    ("flip-tier-8192", 8192, [8192, 5000], [256, 3], 7000, 32, "signed-zeros"),
    ("flip-tier-16384", 16384, [16384], [2048], 15000, 128, "trend"),
    # past 32768 slots: the re-reading kernel's listed path (count and list in one sweep)
    ("stream-40k", 40000, [40000, 33001], [1024, 0], 3072, 128, "normal"),
    ("stream-131k-trend", 131072, [131072], [2048], 4096, 128, "trend"),
    ("stream-70k-ties-straddle", 70000, [70000, 50000], [512, 0], 3072, 64, "ties-straddle"),
    ("stream-70k-signed-zeros", 70000, [70000], [1000], 3072, 128, "signed-zeros"),
    ("stream-70k-infinities", 70000, [70000], [256], 2048, 64, "infinities"),
    ("stream-70k-tie-block", 70000, [70000], [1024], 3072, 128, "tie-block-over-cap"),
    ("stream-70k-crowded-bin", 70000, [70000], [512], 2500, 100, "crowded-bin"),
    ("stream-70k-sample-high", 70000, [70000], [1024], 3072, 128, "stream-sample-high"),
    ("stream-70k-budget-past-list", 70000, [70000], [0], 8000, 64, "normal"),
    # the re-reading kernel's listing from the other end (more than half selected)
    ("stream-flip-70k", 70000, [70000, 50000], [1024, 0], 66000, 128, "ties-straddle"),
    ("stream-flip-70k-signed-zeros", 70000, [70000], [1000], 66000, 128, "signed-zeros"),
    ("stream-flip-70k-infinities", 70000, [70000], [256], 68000, 64, "infinities"),
    ("stream-flip-131k-trend", 131072, [131072], [2048], 127000, 128, "trend"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_select_topk_listed_branches_bit_exact(case):
    name, t_cap, Ts, Ps, B, R, pattern = case
    log(f"[listed topk] {name}")
    L, H = 1, 2
    S = len(Ts)
    sc = _scores(pattern, len(name) * 7919 + t_cap, (L, S, H, t_cap), Ts, Ps, B, R)
    pcap = max(Ps)
    b_cap = max(B, pcap) + 1
    kept, nk = kv.kv_select_topk(torch.from_numpy(sc).to(DEV), _i32(Ts), _i32(Ps), B, R, pcap, b_cap=b_cap)
    kept, nk = kept.cpu().numpy(), nk.cpu().numpy()
    for s in range(S):
        for h in range(H):
            ref = oracle.select_topk(sc[0, s, h], Ts[s], Ps[s], B, R)
            assert nk[s] == ref.size
            assert np.array_equal(kept[0, s, h, :ref.size], ref), f"{name} s{s} h{h}"
            assert np.all(kept[0, s, h, ref.size:] == -1)


RANDOM_CASES = [
    ("random-32k", 32768, [32768, 30001], [1024, 17], 3072, 128),
    ("random-small-share", 32768, [32768], [0], 64, 16),
    ("random-half", 8192, [8192], [0], 4064 + 64, 64),
    ("random-over-half", 8192, [8192], [0], 4065 + 64, 64),
    ("random-empty-sample", 32768, [32768], [30720], 32356, 1536),
    ("random-tier-2048", 2048, [2048, 700], [100, 0], 400, 16),
    # more than half selected: the words to evict listed complemented (tiers up to 16384 slots)
    ("random-flip-2048", 2048, [2048, 700], [100, 0], 1800, 16),
    ("random-flip-4096", 4096, [4096, 2176], [64, 300], 3900, 16),
    ("random-flip-8192", 8192, [8192], [0], 7000, 64),
    ("random-flip-16k", 16384, [16384, 9000], [512, 0], 15000, 64),
    # a budget over half the cache keeps random selection in the 1024 x 32 register tier
    ("random-flip-32k", 32768, [32768, 30001], [1024, 17], 30000, 128),
    # few heads with long caches: the draw split over chunk workgroups (both 1024-thread tiers,
    # ragged lengths, a head that keeps everything)
    ("random-split-16k", 16384, [16384, 9000], [512, 0], 2048, 64),
    ("random-split-ragged-32k", 32768, [32768, 20000, 8000, 100], [1024, 0, 500, 10], 2048, 128),
    ("random-stream-70k", 70000, [70000, 40000], [1024, 0], 3072, 128),
    ("random-stream-131k-small-share", 131072, [131072], [0], 64, 16),
    ("random-stream-70k-budget-past-list", 70000, [70000], [0], 8000, 64),
    # the re-reading kernel's listing from the other end: past the tiers, and a short head of a
    # 32768-slot cache whose budget is half the cache (the 512-thread kernel)
    ("random-stream-flip-70k", 70000, [70000, 40000], [1024, 0], 66000, 128),
    ("random-stream-flip-32k-short", 32768, [20000, 32768], [0, 0], 16384, 64),
]


@pytest.mark.parametrize("with_pos", [False, True])
@pytest.mark.parametrize("case", RANDOM_CASES, ids=[c[0] for c in RANDOM_CASES])
def test_select_random_listed_branches_bit_exact(case, with_pos):
    name, t_cap, Ts, Ps, B, R = case
    log(f"[listed random] {name} pos={with_pos}")
    L, H = 1, 2
    S = len(Ts)
    seed, event = 0x0123456789ABCDEF, 9
    pos = None
    if with_pos:
        pos = np.sort(rng(541, t_cap).integers(0, 2 ** 31 - 1, (L, S, H, t_cap)), axis=-1).astype(np.int32)
    pcap = max(Ps)
    kept, nk = kv.kv_select_random((L, S, H, t_cap), _i32(Ts), _i32(Ps), B, R, pcap, seed, event,
                                   pos=None if pos is None else _i32(pos), b_cap=max(B, pcap))
    kept, nk = kept.cpu().numpy(), nk.cpu().numpy()
    for s in range(S):
        for h in range(H):
            p = None if pos is None else pos[0, s, h]
            ref = oracle.select_random(Ts[s], Ps[s], B, R, p, seed, event, 0, h, s)
            assert nk[s] == ref.size
            assert np.array_equal(kept[0, s, h, :ref.size], ref), f"{name} s{s} h{h}"
            assert np.all(kept[0, s, h, ref.size:] == -1)


UNION_CASES = [
    # name, t_cap, T, P, B, R, G, head pattern, combined pattern
    ("union-listed-32k", 32768, [32768], [1024], 3072, 128, 4, "normal", "ties-straddle"),
    ("union-heads-crowded", 32768, [32768], [512], 2500, 100, 2, "crowded-bin", "normal"),
    ("union-heads-sample-high", 32768, [32768], [1024], 3072, 128, 3, "sample-high", "signed-zeros"),
]


@pytest.mark.parametrize("case", UNION_CASES, ids=[c[0] for c in UNION_CASES])
def test_select_union_listed_branches_bit_exact(case):
    name, t_cap, Ts, Ps, B, R, G, hp, cp = case
    log(f"[listed union] {name}")
    L, H = 1, 2
    S = len(Ts)
    hs = _scores(hp, 11 + t_cap, (L, S, H, G, t_cap), Ts, Ps, B, R)
    comb = _scores(cp, 13 + t_cap, (L, S, H, t_cap), Ts, Ps, B, R)
    pcap = max(Ps)
    kept, nk = kv.kv_select_union(torch.from_numpy(hs).to(DEV), torch.from_numpy(comb).to(DEV), _i32(Ts), _i32(Ps),
                                  B, R, pcap, b_cap=max(B, pcap))
    kept, nk = kept.cpu().numpy(), nk.cpu().numpy()
    for s in range(S):
        for h in range(H):
            ref = oracle.select_union(hs[0, s, h], comb[0, s, h], Ts[s], Ps[s], B, R)
            assert nk[s] == ref.size
            assert np.array_equal(kept[0, s, h, :ref.size], ref), f"{name} s{s} h{h}"
            assert np.all(kept[0, s, h, ref.size:] == -1)


@pytest.mark.parametrize("L", [1, 40])
def test_select_random_split_and_single_workgroup_bit_exact(L):
    # 1 layer x 2 heads takes the split draw; 40 layers x 2 heads (80 heads) one workgroup per head
    log(f"[listed random] L={L}")
    S, H, t_cap, B, R = 1, 2, 32768, 3072, 128
    Ts, Ps = [32768], [1024]
    seed, event = 0x9E3779B97F4A7C15, 3
    kept, nk = kv.kv_select_random((L, S, H, t_cap), _i32(Ts), _i32(Ps), B, R, 1024, seed, event, b_cap=B)
    kept, nk = kept.cpu().numpy(), nk.cpu().numpy()
    for l in range(0, L, 7):
        for h in range(H):
            ref = oracle.select_random(Ts[0], Ps[0], B, R, None, seed, event, l, h, 0)
            assert nk[0] == ref.size
            assert np.array_equal(kept[l, 0, h, :ref.size], ref), f"l{l} h{h}"

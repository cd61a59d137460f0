"""End-to-end GPU parity on the five synthetic workloads (full sizes, launch configuration of bench.py).

Per pass: tri_score -> kv_select_topk -> kv_compact (scored) and
kv_select_random -> kv_compact (random), all through the C ABI.

* Scores: every checked head against the literal fp64 oracle under the 1e-4 rule.
* Kept sets (scored): equal size; differences only at near-threshold slots.
* Kept sets (random): bit-exact.
* Compaction: bit-exact -- against the oracle's gather when the kept sets agree,
  and always as the property K_out[r] == K_in[kept[r]] on every head.
Heads the oracle cannot cover one by one at full size are sampled; every head
is checked for the structural properties (size, order, range, pins, gather).
"""
import numpy as np
import pytest
import torch

import eviction_long_reasoning_amd as kv
import oracle
from parity import (assert_scores, assert_selection_near_threshold, assert_union_near_thresholds, assert_z, keys_f64,
                    log)
from workloads import (centres, kv_numpy, kv_torch, periodic_prompt_torch, periodic_tokens_torch,
                       query_head_centres, query_head_magnitudes, query_magnitudes, workload)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def i32(a):
    return torch.as_tensor(np.asarray(a, np.int32), device=DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


def dev_from_host(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def check_structure(w, kept, nk, Ks, Ko, pos_out, T, P, label, pos_in=None):
    """Properties on every head: size, strict ascent, range, pinned slots, exact gather."""
    L, S, H = kept.shape[:3]
    nk_h = nk.cpu().numpy()
    for s in range(S):
        part = oracle.partition(int(T[s]), int(P[s]), w.budget, w.recent)
        assert nk_h[s] == part.n_kept, f"{label}: n_kept seq {s}"
    n = torch.as_tensor(nk_h.astype(np.int64), device=DEV)[None, :, None, None]
    r = torch.arange(kept.shape[-1], device=DEV)[None, None, None, :]
    valid = r < n
    kk = kept.long()
    assert torch.all(torch.where(valid, kk >= 0, kk == -1)), f"{label}: padding / negative index"
    Tt = torch.as_tensor(np.asarray(T, np.int64), device=DEV)[None, :, None, None]
    assert torch.all(torch.where(valid, kk < Tt, True)), f"{label}: index >= T"
    inc = (kk[..., 1:] > kk[..., :-1]) | ~valid[..., 1:]
    assert torch.all(inc), f"{label}: kept not strictly ascending"
    # pins: the prompt and the clipped recent window are present
    for s in range(S):
        part = oracle.partition(int(T[s]), int(P[s]), w.budget, w.recent)
        if not part.compress:
            continue
        head = kk[:, s, :, :part.n_kept]
        if part.P:
            assert torch.all(head[..., :part.P] == torch.arange(part.P, device=DEV)), f"{label}: prompt seq {s}"
        if part.R:
            assert torch.all(head[..., part.n_kept - part.R:] ==
                             torch.arange(int(T[s]) - part.R, int(T[s]), device=DEV)), f"{label}: recent seq {s}"
    # exact gather, every head (bit comparison on the device)
    idx = torch.where(valid, kk, 0)
    m = min(kept.shape[-1], Ko.shape[3])
    src = torch.take_along_dim(Ks.view(torch.int16) if Ks.dtype == torch.bfloat16 else Ks.view(torch.int32),
                               idx[..., :m, None], dim=3)
    dst = (Ko.view(torch.int16) if Ko.dtype == torch.bfloat16 else Ko.view(torch.int32))[:, :, :, :m]
    ok = (src == dst).all(dim=-1) | ~valid[..., :m]
    assert torch.all(ok), f"{label}: compacted rows differ from K_in[kept]"
    if pos_out is not None:
        want = idx[..., :m].to(torch.int32) if pos_in is None else torch.take_along_dim(pos_in, idx[..., :m], 3)
        assert torch.all((pos_out[..., :m] == want) | ~valid[..., :m]), f"{label}: positions"


def compare_head(w, Kh, Vh, qb, l, s, h, T, P, t, gpu_scores, gpu_kept, Ko, Vo, Po, label, pos=None):
    """Oracle comparison of one head: scores, near-threshold kept rule, gather."""
    kf = keys_f64(Kh[:T], w.dtype)
    ref = oracle.score_literal(kf, None if pos is None else pos[:T], qb[l, h], t, w.theta, w.deltas)
    err = assert_scores(gpu_scores[:T], ref, f"{label} l{l} s{s} h{h}")
    rk = oracle.select_topk(ref, T, P, w.budget, w.recent)
    nd = assert_selection_near_threshold(gpu_kept, rk, ref, T, P, w.budget, w.recent, f"{label} l{l} s{s} h{h}")
    if nd == 0:
        rK, rV, rP = oracle.compact(Kh, Vh, pos, rk)
        assert np.array_equal(Ko[:rk.size], rK) and np.array_equal(Vo[:rk.size], rV)
        assert np.array_equal(Po[:rk.size], rP)
    return err, nd


# --------------------------------------------------------------------------------------------
def test_workload1_tiny_full():
    w = workload(1)
    K, V, _, qb = kv_numpy(w)
    Kd, Vd = torch.from_numpy(K).to(DEV), torch.from_numpy(V).to(DEV)
    sc = kv.tri_score(Kd, torch.from_numpy(qb).to(DEV), i32(w.t_cur), i32(w.seq_len), w.theta, w.deltas)
    kept, nk = kv.kv_select_topk(sc, i32(w.seq_len), i32(w.prompt_len), w.budget, w.recent, w.prompt_cap())
    Ko, Vo, Po = kv.kv_compact(Kd, Vd, kept, nk, i32(w.seq_len), w.out_cap)
    n = int(nk[0])
    err, nd = compare_head(w, K[0, 0, 0], V[0, 0, 0], qb, 0, 0, 0, 512, 64, 512, sc[0, 0, 0].cpu().numpy(),
                           kept[0, 0, 0, :n].cpu().numpy(), Ko[0, 0, 0].cpu().numpy(), Vo[0, 0, 0].cpu().numpy(),
                           Po[0, 0, 0].cpu().numpy(), "tiny")
    log(f"[w1] worst scaled score error {err:.2e}, kept differences {nd}")


def test_workload2_full():
    w = workload(2)
    K, V, _, qb = kv_numpy(w)
    Kd, Vd = dev_from_host(K, w.dtype), dev_from_host(V, w.dtype)
    T, P = w.seq_len, w.prompt_len
    sc = kv.tri_score(Kd, torch.from_numpy(qb).to(DEV), i32(w.t_cur), i32(T), w.theta, w.deltas)
    kept, nk = kv.kv_select_topk(sc, i32(T), i32(P), w.budget, w.recent, w.prompt_cap())
    Ko, Vo, Po = kv.kv_compact(Kd, Vd, kept, nk, i32(T), w.out_cap)
    check_structure(w, kept, nk, Kd, Ko, Po, T, P, "w2")
    sch, kh, Koh, Voh, Poh = sc.cpu().numpy(), kept.cpu().numpy(), host_bits(Ko), host_bits(Vo), Po.cpu().numpy()
    worst, diffs = 0.0, 0
    for h in range(w.n_kv_heads):
        e, nd = compare_head(w, K[0, 0, h], V[0, 0, h], qb, 0, 0, h, int(T[0]), int(P[0]), int(w.t_cur[0]),
                             sch[0, 0, h], kh[0, 0, h, :int(nk[0])], Koh[0, 0, h], Voh[0, 0, h], Poh[0, 0, h], "w2")
        worst, diffs = max(worst, e), diffs + nd
    log(f"[w2] 8 heads: worst scaled score error {worst:.2e}, kept differences {diffs}")
    # random selector, bit-exact on every head
    kr, nkr = kv.kv_select_random((1, 1, 8, w.t_cap), i32(T), i32(P), w.budget, w.recent, w.prompt_cap(), 2, 0)
    kr = kr.cpu().numpy()
    for h in range(8):
        ref = oracle.select_random(int(T[0]), int(P[0]), w.budget, w.recent, None, 2, 0, 0, h, 0)
        assert np.array_equal(kr[0, 0, h, :ref.size], ref)


def test_workload2_shape_at_128k_tokens():
    # the Qwen3-8B-shaped layer at a 131072-token cache: past the selectors' register tiers, so
    # the top-k and random selections run the kernel that re-reads its keys at every step
    w = workload(2, T=131072)
    K, V, _, qb = kv_numpy(w)
    Kd, Vd = dev_from_host(K, w.dtype), dev_from_host(V, w.dtype)
    T, P = w.seq_len, w.prompt_len
    sc = kv.tri_score(Kd, torch.from_numpy(qb).to(DEV), i32(w.t_cur), i32(T), w.theta, w.deltas)
    kept, nk = kv.kv_select_topk(sc, i32(T), i32(P), w.budget, w.recent, w.prompt_cap())
    Ko, Vo, Po = kv.kv_compact(Kd, Vd, kept, nk, i32(T), w.out_cap)
    check_structure(w, kept, nk, Kd, Ko, Po, T, P, "w2-128k")
    sch, kh, Koh, Voh, Poh = sc.cpu().numpy(), kept.cpu().numpy(), host_bits(Ko), host_bits(Vo), Po.cpu().numpy()
    worst, diffs = 0.0, 0
    for h in range(w.n_kv_heads):
        e, nd = compare_head(w, K[0, 0, h], V[0, 0, h], qb, 0, 0, h, int(T[0]), int(P[0]), int(w.t_cur[0]),
                             sch[0, 0, h], kh[0, 0, h, :int(nk[0])], Koh[0, 0, h], Voh[0, 0, h], Poh[0, 0, h],
                             "w2-128k")
        worst, diffs = max(worst, e), diffs + nd
        # the selector on the GPU's own scores is bit-exact
        assert np.array_equal(kh[0, 0, h, :int(nk[0])],
                              oracle.select_topk(sch[0, 0, h], int(T[0]), int(P[0]), w.budget, w.recent))
    log(f"[w2-128k] 8 heads: worst scaled score error {worst:.2e}, kept differences {diffs}")
    kr, _ = kv.kv_select_random((1, 1, 8, w.t_cap), i32(T), i32(P), w.budget, w.recent, w.prompt_cap(), 3, 1)
    kr = kr.cpu().numpy()
    for h in range(8):
        ref = oracle.select_random(int(T[0]), int(P[0]), w.budget, w.recent, None, 3, 1, 0, h, 0)
        assert np.array_equal(kr[0, 0, h, :ref.size], ref)


def test_workload2_full_score_with_norm_term():
    # the full TriAttention score (S_trig + S_norm) on the Qwen3-8B-shaped layer
    w = workload(2)
    K, V, _, qb = kv_numpy(w)
    qabs = query_magnitudes(w, qb)
    Kd, Vd = dev_from_host(K, w.dtype), dev_from_host(V, w.dtype)
    T, P = w.seq_len, w.prompt_len
    sc = kv.tri_score(Kd, torch.from_numpy(qb).to(DEV), i32(w.t_cur), i32(T), w.theta, w.deltas,
                      qabs=torch.from_numpy(qabs).to(DEV))
    kept, nk = kv.kv_select_topk(sc, i32(T), i32(P), w.budget, w.recent, w.prompt_cap())
    sch, kh = sc.cpu().numpy(), kept.cpu().numpy()
    worst, diffs = 0.0, 0
    for h in range(w.n_kv_heads):
        ref = oracle.score_full(keys_f64(K[0, 0, h], w.dtype), None, qb[0, h], qabs[0, h], int(w.t_cur[0]),
                                w.theta, w.deltas)
        worst = max(worst, assert_scores(sch[0, 0, h], ref, f"w2+norm h{h}"))
        rk = oracle.select_topk(ref, int(T[0]), int(P[0]), w.budget, w.recent)
        diffs += assert_selection_near_threshold(kh[0, 0, h, :int(nk[0])], rk, ref, int(T[0]), int(P[0]),
                                                 w.budget, w.recent, f"w2+norm h{h}")
    log(f"[w2+norm] 8 heads: worst scaled score error {worst:.2e}, kept differences {diffs}")


def test_workload2_prefill_compression():
    # the TriAttention engine option that lets prefill tokens compete too: prompt_len = 0, so the
    # whole cache outside the recent window is scored and selected
    w = workload(2)
    K, V, _, qb = kv_numpy(w)
    Kd = dev_from_host(K, w.dtype)
    T = w.seq_len
    P0 = np.zeros_like(w.prompt_len)
    sc = kv.tri_score(Kd, torch.from_numpy(qb).to(DEV), i32(w.t_cur), i32(T), w.theta, w.deltas)
    kept, nk = kv.kv_select_topk(sc, i32(T), i32(P0), w.budget, w.recent, 0)
    assert int(nk[0]) == w.budget
    sch, kh = sc.cpu().numpy(), kept.cpu().numpy()
    diffs, low = 0, 0
    for h in range(w.n_kv_heads):
        ref = oracle.score_literal(keys_f64(K[0, 0, h], w.dtype), None, qb[0, h], int(w.t_cur[0]), w.theta, w.deltas)
        rk = oracle.select_topk(ref, int(T[0]), 0, w.budget, w.recent)
        diffs += assert_selection_near_threshold(kh[0, 0, h, :w.budget], rk, ref, int(T[0]), 0, w.budget, w.recent,
                                                 f"w2-prefill h{h}")
        low += int(np.sum(kh[0, 0, h, :w.budget] < int(w.prompt_len[0])))
    log(f"[w2-prefill] 8 heads: kept differences {diffs}; slots kept from the former prompt range {low}")


def test_workload2_gqa_zscore_max():
    # the GQA rule on the Qwen3-8B-shaped layer: 4 query heads per KV head, each with its own
    # centre, z-normalised per query head over the 32768 keys, max over the group; with and
    # without the norm-based term
    w = workload(2)
    K, V, _, _ = kv_numpy(w)
    nu = query_head_centres(w)
    qabs = query_head_magnitudes(w, nu)
    Kd = dev_from_host(K, w.dtype)
    T, P = w.seq_len, w.prompt_len
    for with_norm in (False, True):
        sc, hs = kv.tri_score_gqa(Kd, torch.from_numpy(nu).to(DEV), i32(w.t_cur), i32(T), w.theta, w.deltas,
                                  qabs=torch.from_numpy(qabs).to(DEV) if with_norm else None)
        kept, nk = kv.kv_select_topk(sc, i32(T), i32(P), w.budget, w.recent, w.prompt_cap())
        # union-based selection on the same scores: per-query-head top-k (k = ceil(n_sel / G)),
        # final choice and top-up by the max of the z-scores
        ukept, unk = kv.kv_select_union(hs, sc, i32(T), i32(P), w.budget, w.recent, w.prompt_cap())
        sch, hsh, kh, ukh = sc.cpu().numpy(), hs.cpu().numpy(), kept.cpu().numpy(), ukept.cpu().numpy()
        worst_s = worst_z = 0.0
        diffs = udiffs = 0
        for h in range(w.n_kv_heads):
            zref, per = oracle.score_gqa(keys_f64(K[0, 0, h], w.dtype), None, nu[0, h], int(w.t_cur[0]), w.theta,
                                         w.deltas, qabs[0, h] if with_norm else None)
            for g in range(w.group):
                worst_s = max(worst_s, assert_scores(hsh[0, 0, h, g], per[g], f"w2-gqa h{h} g{g}"))
            worst_z = max(worst_z, assert_z(sch[0, 0, h], zref, f"w2-gqa h{h}"))
            rk = oracle.select_topk(zref, int(T[0]), int(P[0]), w.budget, w.recent)
            diffs += assert_selection_near_threshold(kh[0, 0, h, :int(nk[0])], rk, zref, int(T[0]), int(P[0]),
                                                     w.budget, w.recent, f"w2-gqa h{h}")
            # the union rule compounds G + 1 rankings: exact on the GPU's own scores, and against the
            # oracle's scores every differing slot sits near one of the rule's thresholds
            uref = oracle.select_union(per, zref, int(T[0]), int(P[0]), w.budget, w.recent)
            assert int(unk[0]) == uref.size
            udiffs += assert_union_near_thresholds(ukh[0, 0, h, :int(unk[0])], hsh[0, 0, h], sch[0, 0, h], per, zref,
                                                   int(T[0]), int(P[0]), w.budget, w.recent, f"w2-union h{h}")
        log(f"[w2-gqa norm={with_norm}] 8 KV heads x 4 query heads: worst head-score error {worst_s:.2e}, "
            f"worst z error {worst_z:.2e}, kept differences {diffs}; union rule: {udiffs} slots differ")


# --------------------------------------------------------------------------------------------
@pytest.fixture(scope="module")
def full_pass():
    w = workload(3)
    log("[w3] generating the 36x8x8x32768x128 bf16 cache on the device")
    mu, qb, _ = centres(w)
    K, V = kv_torch(w, DEV, mu)
    torch.cuda.synchronize()
    yield w, K, V, qb
    del K, V
    torch.cuda.empty_cache()


SAMPLED_HEADS = [(0, 0, 0), (0, 7, 7), (17, 3, 4), (35, 7, 7), (35, 0, 3), (9, 5, 1)]


def test_workload3_full_pass_scored(full_pass):
    w, K, V, qb = full_pass
    T, P = w.seq_len, w.prompt_len
    seq, plen = i32(T), i32(P)
    sc = kv.tri_score(K, torch.from_numpy(qb).to(DEV), i32(w.t_cur), seq, w.theta, w.deltas)
    kept, nk = kv.kv_select_topk(sc, seq, plen, w.budget, w.recent, w.prompt_cap())
    Ko, Vo, Po = kv.kv_compact(K, V, kept, nk, seq, w.out_cap)
    torch.cuda.synchronize()
    log("[w3] scored pass done; structural checks on all 2304 heads")
    check_structure(w, kept, nk, K, Ko, Po, T, P, "w3")
    check_structure(w, kept, nk, V, Vo, None, T, P, "w3-V")
    # determinism: a second pass is bit-identical
    sc2 = kv.tri_score(K, torch.from_numpy(qb).to(DEV), i32(w.t_cur), seq, w.theta, w.deltas)
    kept2, _ = kv.kv_select_topk(sc2, seq, plen, w.budget, w.recent, w.prompt_cap())
    assert torch.equal(sc.view(torch.int32), sc2.view(torch.int32)) and torch.equal(kept, kept2)
    worst, diffs = 0.0, 0
    for (l, s, h) in SAMPLED_HEADS:
        e, nd = compare_head(w, host_bits(K[l, s, h]), host_bits(V[l, s, h]), qb, l, s, h, int(T[s]), int(P[s]),
                             int(w.t_cur[s]), sc[l, s, h].cpu().numpy(), kept[l, s, h, :int(nk[s])].cpu().numpy(),
                             host_bits(Ko[l, s, h]), host_bits(Vo[l, s, h]), Po[l, s, h].cpu().numpy(), "w3")
        worst, diffs = max(worst, e), diffs + nd
        log(f"[w3] head {(l, s, h)}: scaled error {e:.2e}, kept differences {nd}")
    log(f"[w3] sampled heads: worst scaled score error {worst:.2e}, kept differences {diffs}")


def test_workload3_full_pass_random(full_pass):
    w, K, V, qb = full_pass
    T, P = w.seq_len, w.prompt_len
    seed, event = 0x5EED000000000003, 11
    kept, nk = kv.kv_select_random((w.n_layers, w.n_seq, w.n_kv_heads, w.t_cap), i32(T), i32(P), w.budget,
                                   w.recent, w.prompt_cap(), seed, event)
    Ko, Vo, Po = kv.kv_compact(K, V, kept, nk, i32(T), w.out_cap)
    check_structure(w, kept, nk, K, Ko, Po, T, P, "w3-random")
    kh = kept.cpu().numpy()
    for (l, s, h) in SAMPLED_HEADS + [(1, 1, 1), (20, 6, 2)]:
        ref = oracle.select_random(int(T[s]), int(P[s]), w.budget, w.recent, None, seed, event, l, h, s)
        assert np.array_equal(kh[l, s, h, :ref.size], ref), (l, s, h)
    log("[w3] random pass: sampled heads bit-exact, all heads structurally valid")


def test_workload3_full_size_next_rows(full_pass):
    # the next rows at the full pass's size, in the launch configurations bench.py times, on the
    # sampled heads: the norm term, the same memory read as post-RoPE keys (dense, and through a
    # shuffled block table over a head-major pool), the grouped-query z-score + max with G = 4 and
    # union selection on its outputs, the same rule over the memory read as post-RoPE keys through
    # the shuffled table over a token-major pool; recency on every head
    w, K, V, qb = full_pass
    L, S, H, T, d = K.shape
    Tn, Pn = w.seq_len, w.prompt_len
    seq, plen, tcur = i32(Tn), i32(Pn), i32(w.t_cur)
    qbd = torch.from_numpy(qb).to(DEV)
    qabs = query_magnitudes(w, qb)
    sc_full = kv.tri_score(K, qbd, tcur, seq, w.theta, w.deltas, qabs=torch.from_numpy(qabs).to(DEV))
    sc_rot = kv.tri_score_rotated(K, qbd, tcur, seq, w.theta, w.deltas)
    bs, bps = 16, T // 16
    g = torch.Generator(device="cpu")
    g.manual_seed(7)
    table = torch.randperm(S * bps, generator=g).view(S, bps).to(torch.int32).to(DEV)
    pool = K.view(L, S * bps, H, bs, d)                        # head-major pool over the same memory
    sc_pg = kv.tri_score_rotated(pool, qbd, tcur, seq, w.theta, w.deltas, block_table=table, head_major=True)
    nu = query_head_centres(workload(3, q_mode="group-mean"))
    zmax, head = kv.tri_score_gqa(K, torch.from_numpy(nu).to(DEV), tcur, seq, w.theta, w.deltas)
    ku, nku = kv.kv_select_union(head, zmax, seq, plen, w.budget, w.recent, w.prompt_cap())
    pool_tm = K.view(L, S * bps, bs, H, d)                     # token-major pool over the same memory
    zrot, hrot = kv.tri_score_gqa_rotated(pool_tm, torch.from_numpy(nu).to(DEV), tcur, seq, w.theta, w.deltas,
                                          block_table=table)
    kr, nkr = kv.kv_select_recent((L, S, H, T), seq, plen, w.budget, w.recent, w.prompt_cap())
    torch.cuda.synchronize()
    # recency: every head is the prompt followed by the latest slots
    part = oracle.partition(int(Tn[0]), int(Pn[0]), w.budget, w.recent)
    want = torch.from_numpy(oracle.select_recent(int(Tn[0]), int(Pn[0]), w.budget, w.recent)).to(DEV)
    assert torch.all(nkr == part.n_kept) and torch.all(kr[..., :part.n_kept] == want)
    worst = {"norm": 0.0, "rot": 0.0, "paged": 0.0, "head": 0.0, "z": 0.0, "rot_head": 0.0, "rot_z": 0.0}
    tbl = table.cpu().numpy()
    for (l, s, h) in SAMPLED_HEADS[:4]:
        Tl, t = int(Tn[s]), int(w.t_cur[s])
        kf = keys_f64(host_bits(K[l, s, h, :Tl]), w.dtype)
        ref = oracle.score_full(kf, None, qb[l, h], qabs[l, h], t, w.theta, w.deltas)
        worst["norm"] = max(worst["norm"], assert_scores(sc_full[l, s, h, :Tl].cpu().numpy(), ref, f"norm {l, s, h}"))
        ref = oracle.score_rotated(kf, qb[l, h], t, w.theta, w.deltas)
        worst["rot"] = max(worst["rot"], assert_scores(sc_rot[l, s, h, :Tl].cpu().numpy(), ref, f"rot {l, s, h}"))
        j = np.arange(Tl)
        rows = pool[l, torch.from_numpy(tbl[s, j // bs].astype(np.int64)).to(DEV), h,
                    torch.from_numpy(j % bs).to(DEV)]
        ref = oracle.score_rotated(keys_f64(host_bits(rows), w.dtype), qb[l, h], t, w.theta, w.deltas)
        worst["paged"] = max(worst["paged"], assert_scores(sc_pg[l, s, h, :Tl].cpu().numpy(), ref, f"paged {l, s, h}"))
        zref, sref = oracle.score_gqa(kf, None, nu[l, h], t, w.theta, w.deltas)
        hh = head[l, s, h, :, :Tl].cpu().numpy()
        for gq in range(w.group):
            worst["head"] = max(worst["head"], assert_scores(hh[gq], sref[gq], f"gqa {l, s, h} g{gq}"))
        zz = zmax[l, s, h, :Tl].cpu().numpy()
        worst["z"] = max(worst["z"], assert_z(zz, zref, f"gqa z {l, s, h}"))
        # union selection on the kernel's own scores is bit-exact
        uref = oracle.select_union(hh, zz, Tl, int(Pn[s]), w.budget, w.recent)
        assert int(nku[s]) == uref.size
        assert np.array_equal(ku[l, s, h, :uref.size].cpu().numpy(), uref), f"union {l, s, h}"
        rows = pool_tm[l, torch.from_numpy(tbl[s, j // bs].astype(np.int64)).to(DEV),
                       torch.from_numpy(j % bs).to(DEV), h]
        zref, sref = oracle.score_gqa_rotated(keys_f64(host_bits(rows), w.dtype), nu[l, h], t, w.theta, w.deltas)
        hh = hrot[l, s, h, :, :Tl].cpu().numpy()
        for gq in range(w.group):
            worst["rot_head"] = max(worst["rot_head"], assert_scores(hh[gq], sref[gq], f"gqa rot {l, s, h} g{gq}"))
        worst["rot_z"] = max(worst["rot_z"], assert_z(zrot[l, s, h, :Tl].cpu().numpy(), zref, f"gqa rot z {l, s, h}"))
    log(f"[w3-next] sampled heads: worst scaled errors {worst}")


# --------------------------------------------------------------------------------------------
def test_workload5_ragged_scored_vs_random():
    w = workload(5)
    T, P = w.seq_len, w.prompt_len
    log(f"[w5] 128 ragged sequences, sum T = {int(T.sum())}, {int((P > w.budget).sum())} prompts over budget")
    mu, qb, _ = centres(w)
    K, V = kv_torch(w, DEV, mu)
    seq, plen = i32(T), i32(P)
    sc = kv.tri_score(K, torch.from_numpy(qb).to(DEV), i32(w.t_cur), seq, w.theta, w.deltas)
    ks, nks = kv.kv_select_topk(sc, seq, plen, w.budget, w.recent, w.prompt_cap())
    Ko, Vo, Po = kv.kv_compact(K, V, ks, nks, seq, w.out_cap)
    check_structure(w, ks, nks, K, Ko, Po, T, P, "w5-scored")
    worst, diffs = 0.0, 0
    rng_s = np.random.default_rng(5)
    seqs = sorted(set([int(np.argmin(T)), int(np.argmax(T)), int(np.argmax(P)), int(np.argmin(P))] +
                      rng_s.choice(w.n_seq, 4, replace=False).tolist()))
    for s in seqs:
        for h in (0, 5):
            e, nd = compare_head(w, host_bits(K[0, s, h]), host_bits(V[0, s, h]), qb, 0, s, h, int(T[s]), int(P[s]),
                                 int(w.t_cur[s]), sc[0, s, h].cpu().numpy(), ks[0, s, h, :int(nks[s])].cpu().numpy(),
                                 host_bits(Ko[0, s, h]), host_bits(Vo[0, s, h]), Po[0, s, h].cpu().numpy(), "w5")
            worst, diffs = max(worst, e), diffs + nd
    log(f"[w5] scored: sampled {len(seqs)} seqs x 2 heads, worst scaled error {worst:.2e}, kept diffs {diffs}")
    kr, nkr = kv.kv_select_random((1, w.n_seq, w.n_kv_heads, w.t_cap), seq, plen, w.budget, w.recent,
                                  w.prompt_cap(), w.seed_random, 0)
    Kro, Vro, Pro = kv.kv_compact(K, V, kr, nkr, seq, w.out_cap)
    check_structure(w, kr, nkr, K, Kro, Pro, T, P, "w5-random")
    krh, ksh = kr.cpu().numpy(), ks.cpu().numpy()
    jac = []
    for s in range(w.n_seq):
        for h in range(w.n_kv_heads):
            ref = oracle.select_random(int(T[s]), int(P[s]), w.budget, w.recent, None, w.seed_random, 0, 0, h, s)
            assert np.array_equal(krh[0, s, h, :ref.size], ref), (s, h)
            a, b = set(ksh[0, s, h, :ref.size].tolist()), set(ref.tolist())
            jac.append(len(a & b) / max(1, len(a | b)))
    log(f"[w5] random: all 1024 heads bit-exact; mean Jaccard(scored, random) = {np.mean(jac):.3f}")


# --------------------------------------------------------------------------------------------
class _OracleHead:
    """The oracle's own trajectory of one (layer, seq, head) through the periodic workload."""

    def __init__(self, K0, V0, P):
        self.K, self.V = K0[:P].copy(), V0[:P].copy()
        self.pos = np.arange(P, dtype=np.int32)

    def append(self, Kn, Vn, pn):
        self.K = np.concatenate([self.K, Kn])
        self.V = np.concatenate([self.V, Vn])
        self.pos = np.concatenate([self.pos, pn.astype(np.int32)])


@pytest.mark.parametrize("mode", ["scored", "random", "gqa", "random-inplace"])
def test_workload4_periodic_events(mode):
    # gqa: the z-score + max rule over the 8 query heads of each KV head, first 64 events;
    # random-inplace: random eviction with in-place hole filling instead of the gather
    w = workload(4)
    n_events = 64 if mode == "gqa" else w.n_events
    inplace = mode == "random-inplace"
    L, S, H, Tc, d = w.n_layers, w.n_seq, w.n_kv_heads, w.t_cap, w.head_dim
    P = w.prompt_len.astype(np.int64)
    mu0, qb, dr = centres(w)
    K0, V0 = periodic_prompt_torch(w, mu0, dr, DEV)
    bufs = [(K0, V0, torch.arange(Tc, dtype=torch.int32, device=DEV).expand(L, S, H, Tc).contiguous()),
            (torch.empty_like(K0), torch.empty_like(V0), torch.empty((L, S, H, Tc), dtype=torch.int32, device=DEV))]
    cur = 0
    T = P.copy()
    sampled = [(0, int(np.argmin(P)), 0), (23, int(np.argmax(P)), 7), (11, 5, 3), (5, 40, 6)]
    ora = {k: _OracleHead(host_bits(K0[k]), host_bits(V0[k]), int(P[k[1]])) for k in sampled}
    diverged = set()
    qbd = torch.from_numpy(qb).to(DEV)
    if mode == "gqa":
        nu = query_head_centres(w)
        nud = torch.from_numpy(nu).to(DEV)
        gq_out = torch.empty((L, S, H, Tc), dtype=torch.float32, device=DEV)
        gq_head = torch.empty((L, S, H, w.group, Tc), dtype=torch.float32, device=DEV)
        gq_ws = torch.empty((kv.gqa_workspace_bytes(L, S, H, Tc, d, K0.dtype, w.group),), dtype=torch.uint8,
                            device=DEV)
    worst, compared, near = 0.0, 0, 0
    for ev in range(1, n_events + 1):
        Kc, Vc, Pc = bufs[cur]
        Kn, Vn, pn = periodic_tokens_torch(w, ev, (P + w.new_per_event * (ev - 1)).astype(np.int32), mu0, dr, DEV)
        for s in range(S):
            t0 = int(T[s])
            Kc[:, s, :, t0:t0 + w.new_per_event] = Kn[:, s]
            Vc[:, s, :, t0:t0 + w.new_per_event] = Vn[:, s]
            Pc[:, s, :, t0:t0 + w.new_per_event] = pn[s][None, None, :]
        T = T + w.new_per_event
        t_cur = (P + w.new_per_event * ev).astype(np.int32)
        for k in sampled:
            l, s, h = k
            ora[k].append(host_bits(Kn[l, s, h]), host_bits(Vn[l, s, h]), pn[s].cpu().numpy())
        seq = i32(T)
        if mode == "scored":
            sc = kv.tri_score(Kc, qbd, i32(t_cur), seq, w.theta, w.deltas, pos=Pc)
            kept, nk = kv.kv_select_topk(sc, seq, i32(P), w.budget, w.recent, w.prompt_cap())
        elif mode == "gqa":
            sc, _ = kv.tri_score_gqa(Kc, nud, i32(t_cur), seq, w.theta, w.deltas, pos=Pc, out=gq_out,
                                     head_out=gq_head, workspace=gq_ws)
            kept, nk = kv.kv_select_topk(sc, seq, i32(P), w.budget, w.recent, w.prompt_cap())
        else:
            kept, nk = kv.kv_select_random((L, S, H, Tc), seq, i32(P), w.budget, w.recent, w.prompt_cap(),
                                           w.seed_random, ev, pos=Pc)
        if inplace:
            kv.kv_compact_inplace(Kc, Vc, kept, nk, seq, pos=Pc)
            Ko, Vo, Po = Kc, Vc, Pc
        else:
            Ko, Vo, Po = bufs[1 - cur]
            kv.kv_compact(Kc, Vc, kept, nk, seq, Tc, pos=Pc, K_out=Ko, V_out=Vo, pos_out=Po)
        if not inplace and (ev in (1, 2, 64, 256) or ev % 32 == 0):
            check_structure(w, kept, nk, Kc, Ko, Po, T, P, f"w4-{mode} ev{ev}", pos_in=Pc)
        nk_h = nk.cpu().numpy()
        for k in sampled:
            l, s, h = k
            o = ora[k]
            Tn = int(T[s])
            if mode.startswith("random"):
                rk = oracle.select_random(Tn, int(P[s]), w.budget, w.recent, o.pos, w.seed_random, ev, l, h, s)
                gk = kept[l, s, h, :int(nk_h[s])].cpu().numpy()
                assert np.array_equal(gk, rk), (ev, k)
            else:
                if k in diverged:
                    rk = oracle.select_topk(np.zeros(Tn), Tn, int(P[s]), w.budget, w.recent)  # keeps sizes only
                else:
                    if mode == "gqa":
                        ref, _ = oracle.score_gqa(keys_f64(o.K, w.dtype), o.pos, nu[l, h], int(t_cur[s]), w.theta,
                                                  w.deltas)
                        worst = max(worst, assert_z(sc[l, s, h, :Tn].cpu().numpy(), ref, f"w4-gqa ev{ev} {k}"))
                    else:
                        ref = oracle.score_literal(keys_f64(o.K, w.dtype), o.pos, qb[l, h], int(t_cur[s]), w.theta,
                                                   w.deltas)
                        worst = max(worst, assert_scores(sc[l, s, h, :Tn].cpu().numpy(), ref, f"w4 ev{ev} {k}"))
                    rk = oracle.select_topk(ref, Tn, int(P[s]), w.budget, w.recent)
                    gk = kept[l, s, h, :int(nk_h[s])].cpu().numpy()
                    nd = assert_selection_near_threshold(gk, rk, ref, Tn, int(P[s]), w.budget, w.recent,
                                                         f"w4 ev{ev} {k}")
                    compared += 1
                    if nd:
                        near += nd
                        diverged.add(k)   # the trajectories legitimately part here
            if k in diverged and not mode.startswith("random"):
                continue
            if inplace:
                rK, rV, rP, _ = oracle.compact_holes(o.K, o.V, o.pos, rk)
            else:
                rK, rV, rP = oracle.compact(o.K, o.V, o.pos, rk)
            n = rk.size
            assert np.array_equal(host_bits(Ko[l, s, h, :n]), rK) and np.array_equal(host_bits(Vo[l, s, h, :n]), rV)
            assert np.array_equal(Po[l, s, h, :n].cpu().numpy(), rP), (ev, k)
            o.K, o.V, o.pos = rK, rV, rP
        T = nk_h.astype(np.int64)
        if not inplace:
            cur = 1 - cur
        if ev % 32 == 0:
            log(f"[w4-{mode}] event {ev}/{n_events}: cache {int(T.min())}..{int(T.max())} per head")
    if not mode.startswith("random"):
        log(f"[w4-{mode}] {compared} head-events compared, worst scaled error {worst:.2e}, "
            f"near-threshold swaps {near}, diverged heads {len(diverged)}")

"""GPU parity of each kernel against the oracle, at sizes the oracle finishes in seconds.

All calls go through the C ABI (the torch binding only marshals pointers).
Inputs come from the seeded generators in ``workloads``; expected values
come from ``oracle``.
"""
import zlib

import numpy as np
import pytest
import torch

import eviction_long_reasoning_amd as kv
import oracle
from parity import assert_scores, assert_z, keys_f64, log
from workloads import bf16_bits, random_kept, random_scores, rng

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _to_dev_keys(Kf32: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        bits = bf16_bits(Kf32)
        return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(Kf32, np.float32)).to(DEV)


def _host_keys(Kdev: torch.Tensor, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return Kdev.view(torch.int16).cpu().numpy().view(np.uint16)
    return Kdev.cpu().numpy()


def _i32(x) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, np.int32), device=DEV)


# ------------------------------------------------------------------ score ----
SCORE_CASES = [
    # name, dtype, d, L, S, H, T per seq, t_cap, theta, deltas, positions, t offsets
    ("tiny-fp32-d64", "f32", 64, 1, 1, 1, [512], 512, 1e4, [2 ** i for i in range(7)], "slots", [0]),
    ("bf16-d128-ragged", "bf16", 128, 2, 3, 2, [1, 700, 1000], 1030, 1e6, [2 ** i for i in range(17)], "slots", [0, 5, 0]),
    ("bf16-d64-gappy", "bf16", 64, 2, 2, 3, [2176, 1500], 2176, 1e4, [2 ** i for i in range(17)], "gappy", [128, 0]),
    ("bf16-d8", "bf16", 8, 1, 2, 2, [333, 64], 333, 1e4, [1, 2, 4], "slots", [0, 0]),
    ("bf16-d16", "bf16", 16, 1, 1, 3, [129], 200, 1e6, [1, 8, 64], "slots", [0]),
    ("bf16-d32", "bf16", 32, 1, 1, 1, [1000], 1000, 500.0, [0, 3], "slots", [0]),
    ("bf16-d96-idle-lanes", "bf16", 96, 1, 2, 2, [777, 65], 800, 1e6, [2 ** i for i in range(17)], "slots", [0, 0]),
    ("bf16-d256", "bf16", 256, 1, 1, 2, [600], 640, 1e6, [2 ** i for i in range(17)], "gappy", [10]),
    ("fp32-d4", "f32", 4, 1, 1, 1, [70], 70, 1e4, [1, 2], "slots", [0]),
    ("fp32-d128", "f32", 128, 1, 1, 2, [515], 515, 1e6, [2 ** i for i in range(17)], "slots", [0]),
    ("fp32-d256", "f32", 256, 1, 1, 1, [300], 300, 1e6, [2 ** i for i in range(17)], "gappy", [0]),
    ("empty-seq", "bf16", 128, 1, 2, 1, [0, 130], 130, 1e6, [1, 2], "slots", [0, 0]),
    ("future-keys", "bf16", 64, 1, 1, 1, [256], 256, 1e4, [1, 4], "gappy", [-5000]),
]


def _score_inputs(case, seed):
    name, dtype, d, L, S, H, Ts, t_cap, theta, D, pmode, toff = case
    r = rng(500, seed)
    mu = r.standard_normal((L, H, d))
    K = (mu[:, None, :, None, :] + 0.3 * r.standard_normal((L, S, H, t_cap, d))).astype(np.float32)
    qb = (r.standard_normal((L, H, d)) + 0.1 * r.standard_normal((L, H, d))).astype(np.float32)
    Ts = np.array(Ts, np.int32)
    if pmode == "slots":
        pos = None
        t_cur = Ts + np.array(toff, np.int32)
    else:
        pos = np.zeros((L, S, H, t_cap), np.int32)
        for l in range(L):
            for s in range(S):
                for h in range(H):
                    pos[l, s, h] = np.sort(r.choice(40000, size=t_cap, replace=False))
        t_cur = np.full(S, 40000, np.int32) + np.array(toff, np.int32)
    return K, qb, Ts, pos, t_cur


@pytest.mark.parametrize("case", SCORE_CASES, ids=[c[0] for c in SCORE_CASES])
def test_score_matches_oracle(case):
    name, dtype, d, L, S, H, Ts, t_cap, theta, D, pmode, toff = case
    log(f"[score] {name}")
    K, qb, Ts, pos, t_cur = _score_inputs(case, zlib.crc32(name.encode()) % 1000)
    Kd = _to_dev_keys(K, dtype)
    Kh = keys_f64(_host_keys(Kd, dtype), dtype)
    out = torch.full((L, S, H, t_cap), float("nan"), device=DEV)
    kv.tri_score(Kd, torch.from_numpy(qb).to(DEV), _i32(t_cur), _i32(Ts), theta, D,
                 pos=None if pos is None else _i32(pos), out=out)
    got = out.cpu().numpy()
    worst = 0.0
    for l in range(L):
        for s in range(S):
            for h in range(H):
                T = int(Ts[s])
                p = None if pos is None else pos[l, s, h, :T]
                ref = oracle.score_literal(Kh[l, s, h, :T], p, qb[l, h], int(t_cur[s]), theta, D)
                worst = max(worst, assert_scores(got[l, s, h, :T], ref, f"{name} l{l} s{s} h{h}"))
                assert np.all(np.isnan(got[l, s, h, T:])), "slots beyond T were written"
    log(f"[score] {name}: worst scaled error {worst:.2e}")


NORM_CASES = [c for c in SCORE_CASES if c[0] in ("tiny-fp32-d64", "bf16-d128-ragged", "bf16-d64-gappy",
                                                  "bf16-d96-idle-lanes", "fp32-d128")]


# The largest bf16 d = 128 cache one head may hold: its rows are addressed with 32-bit byte offsets
# (t_cap * 256 bytes plus one batch of look-ahead must stay below 2^31).
MAX_T_CAP_BF16_D128 = ((1 << 31) - (64 << 9)) // 256 - 1


def test_score_at_the_largest_t_cap_matches_oracle_on_sampled_slots():
    d, t_cap, theta, D = 128, MAX_T_CAP_BF16_D128, 1e6, [2 ** i for i in range(17)]
    log(f"[score-max] bf16 d{d} t_cap {t_cap} ({t_cap * d * 2 / 2 ** 30:.2f} GiB of keys)")
    r = rng(560, 1)
    block = (r.standard_normal(d) + 0.3 * r.standard_normal((1 << 16, d))).astype(np.float32)
    qb = r.standard_normal((1, 1, d)).astype(np.float32)
    kb = torch.from_numpy(bf16_bits(block).view(np.int16)).to(DEV)
    reps = -(-t_cap // block.shape[0])
    K = kb.repeat(reps, 1)[:t_cap].contiguous().view(torch.bfloat16).view(1, 1, 1, t_cap, d)
    del kb
    Ts = np.array([t_cap], np.int32)
    t_cur = np.array([t_cap + 3], np.int32)
    out = torch.full((1, 1, 1, t_cap), float("nan"), device=DEV)
    kv.tri_score(K, torch.from_numpy(qb).to(DEV), _i32(t_cur), _i32(Ts), theta, D, out=out)
    sample = np.unique(np.concatenate([np.arange(64), np.arange(t_cap - 256, t_cap),
                                       r.choice(t_cap, size=4096, replace=False)]))
    got = out[0, 0, 0, torch.from_numpy(sample).to(DEV)].cpu().numpy()
    Kh = keys_f64(bf16_bits(block[sample % block.shape[0]]), "bf16")
    ref = oracle.score_literal(Kh, sample.astype(np.int64), qb[0, 0], int(t_cur[0]), theta, D)
    worst = assert_scores(got, ref, "largest t_cap")
    assert not torch.isnan(out).any().item(), "a slot below T was not written"
    log(f"[score-max] {sample.size} sampled slots: worst scaled error {worst:.2e}")


@pytest.mark.parametrize("case", NORM_CASES, ids=[c[0] for c in NORM_CASES])
def test_score_with_norm_term_matches_oracle(case):
    name, dtype, d, L, S, H, Ts, t_cap, theta, D, pmode, toff = case
    log(f"[score+norm] {name}")
    K, qb, Ts, pos, t_cur = _score_inputs(case, zlib.crc32(name.encode()) % 1000)
    r = rng(540, d)
    centre = np.abs(qb[..., 0::2].astype(np.float64) + 1j * qb[..., 1::2])
    qabs = (centre / r.uniform(0.5, 1.0, centre.shape)).astype(np.float32)
    qabs[..., 1] = 0.0                                   # a band without statistics contributes nothing
    Kd = _to_dev_keys(K, dtype)
    Kh = keys_f64(_host_keys(Kd, dtype), dtype)
    out = kv.tri_score(Kd, torch.from_numpy(qb).to(DEV), _i32(t_cur), _i32(Ts), theta, D,
                       pos=None if pos is None else _i32(pos), qabs=torch.from_numpy(qabs).to(DEV))
    got = out.cpu().numpy()
    worst = 0.0
    for l in range(L):
        for s in range(S):
            for h in range(H):
                T = int(Ts[s])
                p = None if pos is None else pos[l, s, h, :T]
                ref = oracle.score_full(Kh[l, s, h, :T], p, qb[l, h], qabs[l, h], int(t_cur[s]), theta, D)
                worst = max(worst, assert_scores(got[l, s, h, :T], ref, f"{name} l{l} s{s} h{h}"))
    log(f"[score+norm] {name}: worst scaled error {worst:.2e}")


GQA_CASES = [
    # name, dtype, d, L, S, H, G, T per seq, t_cap, positions, norm, zero query head
    ("gqa-bf16-d128-g4", "bf16", 128, 1, 2, 2, 4, [1500, 513], 1500, "slots", False, -1),
    ("gqa-bf16-d128-g8-norm", "bf16", 128, 2, 1, 2, 8, [1100], 1100, "slots", True, -1),
    ("gqa-bf16-d64-g8-gappy", "bf16", 64, 1, 2, 3, 8, [2000, 700], 2048, "gappy", False, -1),
    ("gqa-bf16-d64-g7-norm-gappy", "bf16", 64, 1, 1, 2, 7, [999], 1024, "gappy", True, -1),
    ("gqa-bf16-d96-g3", "bf16", 96, 1, 1, 2, 3, [600], 640, "slots", False, 1),
    ("gqa-bf16-d16-g5", "bf16", 16, 1, 2, 1, 5, [300, 1], 300, "slots", False, -1),
    ("gqa-fp32-d64-g2", "f32", 64, 1, 1, 2, 2, [777], 800, "slots", True, 0),
    ("gqa-fp32-d8-g1", "f32", 8, 1, 1, 1, 1, [100], 100, "slots", False, -1),
    ("gqa-bf16-d128-g6-empty", "bf16", 128, 1, 2, 1, 6, [0, 1030], 1030, "slots", False, -1),
    ("gqa-bf16-d256-g16-norm", "bf16", 256, 1, 1, 2, 16, [700], 704, "slots", True, 3),
    ("gqa-fp32-d128-g12-gappy", "f32", 128, 1, 2, 1, 12, [600, 17], 640, "gappy", False, -1),
    ("gqa-bf16-d32-g4-tiny", "bf16", 32, 2, 1, 1, 4, [3], 5, "slots", False, -1),
    # groups of at most four with contiguous positions and bf16 rows of 4, 8 or 16 pieces take the
    # VALU form: G = 1..4, with and without the norm term, a zero query head, ragged tails
    ("gqa-valu-bf16-d64-g2-norm", "bf16", 64, 1, 2, 2, 2, [1500, 1025], 1536, "slots", True, -1),
    ("gqa-valu-bf16-d128-g1", "bf16", 128, 1, 1, 2, 1, [2049], 2100, "slots", False, -1),
    ("gqa-valu-bf16-d128-g3-zero", "bf16", 128, 2, 1, 1, 3, [1030], 1030, "slots", False, 2),
    ("gqa-valu-bf16-d128-g4-norm", "bf16", 128, 1, 2, 1, 4, [3000, 1], 3000, "slots", True, -1),
    ("gqa-valu-bf16-d32-g4", "bf16", 32, 1, 1, 3, 4, [4097], 4100, "slots", False, -1),
]


@pytest.mark.parametrize("case", GQA_CASES, ids=[c[0] for c in GQA_CASES])
def test_gqa_score_matches_oracle(case):
    name, dtype, d, L, S, H, G, Ts, t_cap, pmode, norm, zero_g = case
    log(f"[gqa] {name}")
    seed = zlib.crc32(name.encode()) % 1000
    r = rng(560, seed)
    theta, D = 1e6, [2 ** i for i in range(17)]
    mu = r.standard_normal((L, H, d))
    K = (mu[:, None, :, None, :] + 0.3 * r.standard_normal((L, S, H, t_cap, d))).astype(np.float32)
    nu = r.standard_normal((L, H, G, d)).astype(np.float32)
    if zero_g >= 0:
        nu[:, :, zero_g] = 0.0                       # a query head whose scores are all 0: sigma = 0, z = 0
    Ts = np.array(Ts, np.int32)
    if pmode == "slots":
        pos, t_cur = None, Ts.copy()
    else:
        pos = np.stack([np.sort(r.choice(50000, size=t_cap, replace=False)) for _ in range(L * S * H)])
        pos = pos.reshape(L, S, H, t_cap).astype(np.int32)
        t_cur = np.full(S, 50000, np.int32)
    qabs = None
    if norm:
        centre = np.abs(nu[..., 0::2].astype(np.float64) + 1j * nu[..., 1::2])
        qabs = (centre / r.uniform(0.5, 1.0, centre.shape)).astype(np.float32)
    Kd = _to_dev_keys(K, dtype)
    Kh = keys_f64(_host_keys(Kd, dtype), dtype)
    out = torch.full((L, S, H, t_cap), float("nan"), device=DEV)
    hout = torch.full((L, S, H, G, t_cap), float("nan"), device=DEV)
    ws = torch.full((kv.gqa_workspace_bytes(L, S, H, t_cap, d, Kd.dtype, G),), 0xAB, dtype=torch.uint8, device=DEV)
    kv.tri_score_gqa(Kd, torch.from_numpy(nu).to(DEV), _i32(t_cur), _i32(Ts), theta, D,
                     pos=None if pos is None else _i32(pos), qabs=None if qabs is None else torch.from_numpy(qabs).to(DEV),
                     out=out, head_out=hout, workspace=ws)
    got, ghead = out.cpu().numpy(), hout.cpu().numpy()
    worst_s = worst_z = 0.0
    for l in range(L):
        for s in range(S):
            for h in range(H):
                T = int(Ts[s])
                p = None if pos is None else pos[l, s, h, :T]
                zref, sref = oracle.score_gqa(Kh[l, s, h, :T], p, nu[l, h], int(t_cur[s]), theta, D,
                                              None if qabs is None else qabs[l, h])
                for g in range(G):
                    worst_s = max(worst_s, assert_scores(ghead[l, s, h, g, :T], sref[g], f"{name} l{l} s{s} h{h} g{g}"))
                worst_z = max(worst_z, assert_z(got[l, s, h, :T], zref, f"{name} l{l} s{s} h{h}"))
                assert np.all(np.isnan(got[l, s, h, T:])) and np.all(np.isnan(ghead[l, s, h, :, T:])), \
                    "slots beyond T were written"
    log(f"[gqa] {name}: worst scaled head-score error {worst_s:.2e}, worst z error {worst_z:.2e}")


def test_gqa_is_deterministic():
    # the per-query-head statistics are reduced in a fixed order: repeated calls agree bit for bit
    L, S, H, G, T, d = 1, 1, 4, 8, 4000, 128
    r = rng(561, 0)
    K = _to_dev_keys(r.standard_normal((L, S, H, T, d)).astype(np.float32), "bf16")
    nu = torch.from_numpy(r.standard_normal((L, H, G, d)).astype(np.float32)).to(DEV)
    a, ha = kv.tri_score_gqa(K, nu, _i32([T]), _i32([T]), 1e6, [1, 2, 4])
    for _ in range(3):
        b, hb = kv.tri_score_gqa(K, nu, _i32([T]), _i32([T]), 1e6, [1, 2, 4])
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        assert torch.equal(ha.view(torch.int32), hb.view(torch.int32))


ROT_CASES = [
    # name, dtype, d, L, S, H, T per seq, style, norm, paged block size (0 = dense), head-major pool
    ("rot-bf16-d128-inter", "bf16", 128, 2, 2, 2, [1000, 777], "interleaved", False, 0, False),
    ("rot-bf16-d128-half", "bf16", 128, 1, 2, 3, [1030, 64], "half", False, 0, False),
    ("rot-bf16-d64-half-norm", "bf16", 64, 2, 1, 2, [900], "half", True, 0, False),
    ("rot-bf16-d96-inter-norm", "bf16", 96, 1, 2, 2, [500, 130], "interleaved", True, 0, False),
    ("rot-fp32-d64-half", "f32", 64, 1, 1, 2, [333], "half", False, 0, False),
    ("rot-fp32-d8-inter", "f32", 8, 1, 1, 1, [200], "interleaved", True, 0, False),
    ("rot-paged16-bf16-d128", "bf16", 128, 2, 3, 4, [1000, 1, 517], "interleaved", True, 16, False),
    ("rot-paged64-bf16-d64-half", "bf16", 64, 1, 2, 8, [2000, 1500], "half", False, 64, False),
    ("rot-paged16-headmajor-bf16-d128", "bf16", 128, 2, 3, 4, [1000, 1, 517], "interleaved", True, 16, True),
    ("rot-paged32-headmajor-fp32-d64-half", "f32", 64, 1, 2, 3, [700, 64], "half", False, 32, True),
    # blocks smaller than a wave step's slots (4 at 16 lanes per key, 32 at 2): per-slot rows
    ("rot-paged2-bf16-d96-inter-norm-idle", "bf16", 96, 1, 2, 2, [301, 45], "interleaved", True, 2, False),
    ("rot-paged1-headmajor-bf16-d128-half", "bf16", 128, 1, 2, 2, [130, 77], "half", False, 1, True),
    ("rot-paged8-fp32-d8-norm", "f32", 8, 1, 2, 1, [200, 31], "interleaved", True, 8, False),
    # a block of exactly one step, idle lanes past head_dim 96
    ("rot-paged4-bf16-d96-inter", "bf16", 96, 1, 2, 3, [259, 3], "interleaved", False, 4, False),
    # head_dim 256: 32 lanes per key (two slots a step) and, in fp32, 64 (one slot a step)
    ("rot-bf16-d256-half-norm", "bf16", 256, 1, 2, 2, [300, 77], "half", True, 0, False),
    ("rot-paged1-bf16-d256", "bf16", 256, 1, 2, 2, [300, 77], "interleaved", False, 1, False),
    ("rot-paged2-headmajor-bf16-d256", "bf16", 256, 1, 2, 2, [300, 77], "interleaved", True, 2, True),
    ("rot-fp32-d256-inter", "f32", 256, 1, 2, 2, [300, 77], "interleaved", False, 0, False),
    ("rot-paged1-fp32-d256-half-norm", "f32", 256, 1, 2, 2, [300, 77], "half", True, 1, False),
]


@pytest.mark.parametrize("case", ROT_CASES, ids=[c[0] for c in ROT_CASES])
def test_score_rotated_matches_oracle(case):
    name, dtype, d, L, S, H, Ts, style, norm, bs, hm = case
    log(f"[rotated] {name}")
    r = rng(550, zlib.crc32(name.encode()) % 1000)
    Ts = np.array(Ts, np.int32)
    theta, D = 1e6, [2 ** i for i in range(17)]
    qb = r.standard_normal((L, H, d)).astype(np.float32)
    qabs = None
    if norm:
        re, im = oracle.band_slices(d, style)
        qabs = (np.hypot(qb[..., re], qb[..., im]) / r.uniform(0.6, 1.0, (L, H, d // 2))).astype(np.float32)
    t_cur = (Ts + 7).astype(np.int32)
    if bs == 0:
        t_cap = int(Ts.max()) + 3
        K = (r.standard_normal((L, 1, H, 1, d)) + 0.3 * r.standard_normal((L, S, H, t_cap, d))).astype(np.float32)
        Kd = _to_dev_keys(K, dtype)
        Kh = keys_f64(_host_keys(Kd, dtype), dtype)
        rows = lambda l, s, h, T: Kh[l, s, h, :T]
        out = kv.tri_score_rotated(Kd, torch.from_numpy(qb).to(DEV), _i32(t_cur), _i32(Ts), theta, D, rope_style=style,
                                   qabs=None if qabs is None else torch.from_numpy(qabs).to(DEV))
    else:
        bps = (int(Ts.max()) + bs - 1) // bs
        n_blocks = S * bps + 5
        pool = (r.standard_normal((L, 1, 1, H, d)) + 0.3 * r.standard_normal((L, n_blocks, bs, H, d))).astype(np.float32)
        if hm:
            pool = np.ascontiguousarray(pool.transpose(0, 1, 3, 2, 4))     # [L, n_blocks, H, bs, d]
        table = r.permutation(n_blocks)[:S * bps].reshape(S, bps).astype(np.int32)
        Kd = _to_dev_keys(pool, dtype)
        Ph = keys_f64(_host_keys(Kd, dtype), dtype)
        at = (lambda l, b, o, h: Ph[l, b, h, o]) if hm else (lambda l, b, o, h: Ph[l, b, o, h])
        rows = lambda l, s, h, T: np.stack([at(l, table[s, j // bs], j % bs, h) for j in range(T)]) if T else \
            np.zeros((0, d))
        out = kv.tri_score_rotated(Kd, torch.from_numpy(qb).to(DEV), _i32(t_cur), _i32(Ts), theta, D, rope_style=style,
                                   block_table=_i32(table), qabs=None if qabs is None else torch.from_numpy(qabs).to(DEV),
                                   head_major=hm)
    got = out.cpu().numpy()
    worst = 0.0
    for l in range(L):
        for s in range(S):
            for h in range(H):
                T = int(Ts[s])
                ref = oracle.score_rotated(rows(l, s, h, T), qb[l, h], int(t_cur[s]), theta, D, style=style,
                                           qabs=None if qabs is None else qabs[l, h])
                worst = max(worst, assert_scores(got[l, s, h, :T], ref, f"{name} l{l} s{s} h{h}"))
    log(f"[rotated] {name}: worst scaled error {worst:.2e}")


GQA_ROT_CASES = [
    # name, dtype, d, L, S, H, G, T per seq, style, norm, paged block size (0 = dense), head-major pool
    ("gqa-rot-bf16-d128-g4-inter", "bf16", 128, 2, 2, 2, 4, [1500, 777], "interleaved", False, 0, False),
    ("gqa-rot-bf16-d128-g4-half-norm", "bf16", 128, 1, 2, 2, 4, [1030, 64], "half", True, 0, False),
    ("gqa-rot-paged16-bf16-d128-g8", "bf16", 128, 2, 3, 2, 8, [2000, 1, 517], "interleaved", False, 16, False),
    ("gqa-rot-paged16-hm-bf16-d128-g4-norm", "bf16", 128, 1, 2, 4, 4, [1100, 600], "interleaved", True, 16, True),
    ("gqa-rot-paged64-hm-bf16-d64-g2-half", "bf16", 64, 1, 2, 3, 2, [2100, 900], "half", False, 64, True),
    ("gqa-rot-fp32-d64-g3-norm", "f32", 64, 1, 1, 2, 3, [999], "interleaved", True, 0, False),
    ("gqa-rot-bf16-d96-g1-idle-lanes", "bf16", 96, 1, 1, 2, 1, [700], "interleaved", False, 0, False),
    ("gqa-rot-bf16-d32-g5-empty", "bf16", 32, 1, 2, 1, 5, [0, 1030], "interleaved", False, 32, False),
    # blocks smaller than a wave step's slots: per-slot rows (idle lanes zeroed after the sums)
    ("gqa-rot-paged2-bf16-d96-g4-norm-idle", "bf16", 96, 1, 2, 2, 4, [301, 45], "interleaved", True, 2, False),
    ("gqa-rot-paged1-hm-bf16-d128-g3-half", "bf16", 128, 1, 2, 2, 3, [130, 77], "half", False, 1, True),
    ("gqa-rot-paged2-hm-fp32-d64-g8-norm", "f32", 64, 1, 1, 2, 8, [260], "interleaved", True, 2, True),
    # a block of exactly one step, idle lanes past head_dim 96
    ("gqa-rot-paged4-bf16-d96-g2", "bf16", 96, 1, 2, 3, 2, [259, 3], "interleaved", False, 4, False),
]


@pytest.mark.parametrize("case", GQA_ROT_CASES, ids=[c[0] for c in GQA_ROT_CASES])
def test_gqa_rotated_matches_oracle(case):
    name, dtype, d, L, S, H, G, Ts, style, norm, bs, hm = case
    log(f"[gqa-rot] {name}")
    r = rng(551, zlib.crc32(name.encode()) % 1000)
    Ts = np.array(Ts, np.int32)
    theta, D = 1e6, [2 ** i for i in range(17)]
    nu = r.standard_normal((L, H, G, d)).astype(np.float32)
    qabs = None
    if norm:
        re, im = oracle.band_slices(d, style)
        qabs = (np.hypot(nu[..., re], nu[..., im]) / r.uniform(0.6, 1.0, (L, H, G, d // 2))).astype(np.float32)
    t_cur = (Ts + 7).astype(np.int32)
    kw = dict(rope_style=style, qabs=None if qabs is None else torch.from_numpy(qabs).to(DEV))
    if bs == 0:
        t_cap = int(Ts.max()) + 3
        K = (r.standard_normal((L, 1, H, 1, d)) + 0.3 * r.standard_normal((L, S, H, t_cap, d))).astype(np.float32)
        Kd = _to_dev_keys(K, dtype)
        Kh = keys_f64(_host_keys(Kd, dtype), dtype)
        rows = lambda l, s, h, T: Kh[l, s, h, :T]
    else:
        bps = (int(Ts.max()) + bs - 1) // bs
        t_cap = bps * bs
        n_blocks = S * bps + 5
        pool = (r.standard_normal((L, 1, 1, H, d)) + 0.3 * r.standard_normal((L, n_blocks, bs, H, d))).astype(np.float32)
        if hm:
            pool = np.ascontiguousarray(pool.transpose(0, 1, 3, 2, 4))     # [L, n_blocks, H, bs, d]
        table = r.permutation(n_blocks)[:S * bps].reshape(S, bps).astype(np.int32)
        Kd = _to_dev_keys(pool, dtype)
        Ph = keys_f64(_host_keys(Kd, dtype), dtype)
        at = (lambda l, b, o, h: Ph[l, b, h, o]) if hm else (lambda l, b, o, h: Ph[l, b, o, h])
        rows = lambda l, s, h, T: np.stack([at(l, table[s, j // bs], j % bs, h) for j in range(T)]) if T else \
            np.zeros((0, d))
        kw.update(block_table=_i32(table), head_major=hm)
    out = torch.full((L, S, H, t_cap), float("nan"), device=DEV)
    hout = torch.full((L, S, H, G, t_cap), float("nan"), device=DEV)
    kv.tri_score_gqa_rotated(Kd, torch.from_numpy(nu).to(DEV), _i32(t_cur), _i32(Ts), theta, D, out=out,
                             head_out=hout, **kw)
    got, ghead = out.cpu().numpy(), hout.cpu().numpy()
    worst_s = worst_z = 0.0
    for l in range(L):
        for s in range(S):
            for h in range(H):
                T = int(Ts[s])
                if T == 0:
                    assert np.all(np.isnan(got[l, s, h])), "an empty sequence was written"
                    continue
                zref, sref = oracle.score_gqa_rotated(rows(l, s, h, T), nu[l, h], int(t_cur[s]), theta, D, style,
                                                      None if qabs is None else qabs[l, h])
                for g in range(G):
                    worst_s = max(worst_s, assert_scores(ghead[l, s, h, g, :T], sref[g], f"{name} l{l} s{s} h{h} g{g}"))
                worst_z = max(worst_z, assert_z(got[l, s, h, :T], zref, f"{name} l{l} s{s} h{h}"))
                assert np.all(np.isnan(got[l, s, h, T:])) and np.all(np.isnan(ghead[l, s, h, :, T:]))
    log(f"[gqa-rot] {name}: worst scaled head-score error {worst_s:.2e}, worst z error {worst_z:.2e}")


def test_score_deterministic():
    case = SCORE_CASES[1]
    K, qb, Ts, pos, t_cur = _score_inputs(case, 7)
    Kd = _to_dev_keys(K, "bf16")
    args = (Kd, torch.from_numpy(qb).to(DEV), _i32(t_cur), _i32(Ts), 1e6, [2 ** i for i in range(17)])
    a = kv.tri_score(*args).cpu().numpy()
    b = kv.tri_score(*args).cpu().numpy()
    T = Ts[:, None]
    mask = np.arange(a.shape[-1])[None, :] < T
    for l in range(a.shape[0]):
        for h in range(a.shape[2]):
            assert np.array_equal(a[l, :, h][mask].view(np.uint32), b[l, :, h][mask].view(np.uint32))


# ----------------------------------------------------------------- select ----
SELECT_CASES = [
    # name, t_cap, T per seq, P per seq, B, R, score kind
    ("tier-1k", 1000, [1000, 999, 700, 5], [10, 0, 690, 0], 300, 16, "ties"),
    ("tier-4k", 4096, [4096, 3000, 2049], [100, 2500, 1000], 2048, 128, "specials"),
    ("tier-8k", 8192, [8192, 8000], [512, 0], 2048, 128, "ties"),
    ("tier-16k", 16000, [16000, 12345], [1024, 77], 3072, 128, "normal"),
    ("tier-32k", 32768, [32768, 32767, 20000], [1024, 512, 4096], 3072, 128, "normal"),
    ("tier-64k", 65536, [65536, 40000], [1024, 0], 2048, 64, "ties"),
    ("concentrated", 5000, [5000, 5000], [64, 64], 1000, 16, "concentrated"),
    ("all-equal", 3000, [3000], [100], 500, 10, "equal"),
    ("prompt-over-budget", 3000, [3000, 2500], [2500, 2049], 2048, 128, "normal"),
    ("recent-clipped", 3000, [3000], [2000], 2048, 128, "normal"),
    ("fits-budget", 3000, [2048, 100], [100, 50], 2048, 128, "normal"),
    ("no-recent", 777, [777], [0], 100, 0, "specials"),
    ("huge-range", 4000, [4000, 3000], [10, 10], 1000, 8, "huge"),
    ("ulp-range", 4000, [4000], [10], 1500, 8, "ulp"),
    ("denormals", 2500, [2500], [0], 300, 4, "denormal"),
    ("inf-mix", 6000, [6000, 5000], [32, 0], 2048, 64, "infmix"),
    # past 65536 slots: the kernel that re-reads its keys at every step
    ("stream-70k-specials", 70000, [70000, 65537, 3000], [1024, 0, 100], 3072, 128, "specials"),
    ("stream-128k", 131072, [131072, 100001], [2048, 4096], 4096, 128, "normal"),
    ("stream-96k-ties", 98304, [98304, 80000], [512, 0], 3072, 64, "ties"),
    ("stream-80k-concentrated", 80000, [80000], [64], 2048, 16, "concentrated"),
    ("stream-66k-infmix", 66000, [66000, 66000], [32, 0], 2048, 64, "infmix"),
    ("stream-66k-huge", 66000, [66000], [10], 1000, 8, "huge"),
    ("stream-70k-equal", 70000, [70000], [100], 500, 10, "equal"),
    ("stream-70k-prompt-over-budget", 70000, [70000, 69000], [2500, 2049], 2048, 128, "normal"),
    # the threshold's value bin holds thousands of keys: the radix passes resolve it
    ("crowded-bin", 20000, [20000, 15000], [100, 0], 3000, 64, "cluster"),
    ("stream-70k-crowded-bin", 70000, [70000], [100], 3000, 64, "cluster"),
]


def _select_scores(name, kind, shape):
    seed = zlib.crc32(name.encode()) % 10000
    if kind == "ties":
        return random_scores(seed, shape, ties=0.4)
    if kind == "specials":
        return random_scores(seed, shape, ties=0.1, specials=True)
    if kind == "concentrated":
        x = random_scores(seed, shape)
        return (np.float32(1000.0) + np.float32(1e-3) * x).astype(np.float32)
    if kind == "equal":
        return np.full(shape, 3.25, np.float32)
    if kind == "huge":      # value range overflows fp32: the value-binned pass must stand aside
        x = random_scores(seed, shape)
        x.reshape(-1)[::7] = np.float32(3.0e38)
        x.reshape(-1)[3::7] = np.float32(-3.0e38)
        return x
    if kind == "ulp":       # distinct values a few ulps apart around 1.0
        n = int(np.prod(shape))
        r = rng(530, seed)
        bits = (np.float32(1.0).view(np.uint32) + r.integers(0, 4 * n, n).astype(np.uint32))
        return bits.view(np.float32).reshape(shape)
    if kind == "denormal":  # range narrower than any normal float
        n = int(np.prod(shape))
        r = rng(531, seed)
        return r.integers(0, 0x7FFFF, n).astype(np.uint32).view(np.float32).reshape(shape)
    if kind == "cluster":   # outliers stretch the value range: the threshold's bin is crowded
        n = int(np.prod(shape))
        r = rng(532, seed)
        x = (np.float32(1.0) + np.float32(1e-3) * r.random(n, dtype=np.float32)).astype(np.float32)
        x[::97] = np.float32(1e6)
        x[1::101] = np.float32(-1e6)
        return x.reshape(shape)
    if kind == "infmix":
        x = random_scores(seed, shape, ties=0.05)
        flat = x.reshape(-1)
        flat[::5] = np.inf
        flat[2::9] = -np.inf
        flat[4::11] = np.nan
        return x
    return random_scores(seed, shape)


@pytest.mark.parametrize("case", SELECT_CASES, ids=[c[0] for c in SELECT_CASES])
def test_select_topk_bit_exact(case):
    name, t_cap, Ts, Ps, B, R, kind = case
    log(f"[select] {name}")
    L, H = 2, 2
    S = len(Ts)
    sc = _select_scores(name, kind, (L, S, H, t_cap))
    pcap = max(Ps)
    b_cap = max(B, pcap) + 3
    kept, nk = kv.kv_select_topk(torch.from_numpy(sc).to(DEV), _i32(Ts), _i32(Ps), B, R, pcap, b_cap=b_cap)
    kept = kept.cpu().numpy()
    nk = nk.cpu().numpy()
    for s in range(S):
        ref_n = oracle.partition(Ts[s], Ps[s], B, R).n_kept
        assert nk[s] == ref_n
        for l in range(L):
            for h in range(H):
                ref = oracle.select_topk(sc[l, s, h], Ts[s], Ps[s], B, R)
                assert np.array_equal(kept[l, s, h, :ref_n], ref), f"{name} l{l} s{s} h{h}"
                assert np.all(kept[l, s, h, ref_n:] == -1)


@pytest.mark.parametrize("case", SELECT_CASES[:6] + SELECT_CASES[8:], ids=[c[0] for c in SELECT_CASES[:6] + SELECT_CASES[8:]])
@pytest.mark.parametrize("with_pos", [False, True])
def test_select_random_bit_exact(case, with_pos):
    name, t_cap, Ts, Ps, B, R, _ = case
    log(f"[random] {name} pos={with_pos}")
    L, H = 2, 3
    S = len(Ts)
    seed, event = 0xDEADBEEF12345678, 77
    pos = None
    if with_pos:
        r = rng(510, t_cap)
        pos = np.sort(r.integers(0, 2 ** 31 - 1, (L, S, H, t_cap)), axis=-1).astype(np.int32)
    pcap = max(Ps)
    kept, nk = kv.kv_select_random((L, S, H, t_cap), _i32(Ts), _i32(Ps), B, R, pcap, seed, event,
                                   pos=None if pos is None else _i32(pos))
    kept = kept.cpu().numpy()
    nk = nk.cpu().numpy()
    for s in range(S):
        for l in range(L):
            for h in range(H):
                p = None if pos is None else pos[l, s, h]
                ref = oracle.select_random(Ts[s], Ps[s], B, R, p, seed, event, l, h, s)
                assert nk[s] == ref.size
                assert np.array_equal(kept[l, s, h, :ref.size], ref), f"{name} l{l} s{s} h{h}"
                assert np.all(kept[l, s, h, ref.size:] == -1)


# Positions that run consecutively from a multiple of 4 let a group of 512 slots share 128 Philox
# blocks (each lane draws some and passes words to the lanes that need them); any other layout
# draws per slot. Layouts: runs from offsets 0..3 (only 0 and 4 share), a run broken once inside a
# group, runs restarting every 300 slots, and the slots themselves; every tier from the 256-thread
# one to the re-reading kernel, budgets below and above half the cache.
@pytest.mark.parametrize("t_cap,budget", [(2048, 500), (2176, 1900), (8192, 3000), (16384, 9000),
                                          (32768, 20000), (32768, 3072), (70000, 20000)])
def test_select_random_block_sharing_layouts(t_cap, budget):
    L, S, H = 1, 7, 2
    Ts = [t_cap, t_cap - 5, t_cap, t_cap, t_cap - 77, t_cap, t_cap]
    Ps = [64, 37, 1, 130, 0, 1000, 3]
    R = 128
    pcap = max(Ps)
    base = np.arange(t_cap, dtype=np.int64)
    layouts = [base + 40, base + 41, base + 42, base + 7, base + 4 * 1000,
               np.where(base < 700, base, base + 9), (base // 300) * 1000 + base % 300]
    pos = np.zeros((L, S, H, t_cap), np.int32)
    for s in range(S):
        pos[0, s, :] = layouts[s]
    seed, event = 0x0123456789ABCDEF, 5
    log(f"[random blocks] t_cap {t_cap} budget {budget}")
    for with_pos in (True, False):
        kept, nk = kv.kv_select_random((L, S, H, t_cap), _i32(Ts), _i32(Ps), budget, R, pcap, seed, event,
                                       pos=_i32(pos) if with_pos else None)
        kept, nk = kept.cpu().numpy(), nk.cpu().numpy()
        for s in range(S):
            for h in range(H):
                ref = oracle.select_random(Ts[s], Ps[s], budget, R, pos[0, s, h] if with_pos else None,
                                           seed, event, 0, h, s)
                assert nk[s] == ref.size
                assert np.array_equal(kept[0, s, h, :ref.size], ref), f"t_cap {t_cap} s{s} h{h} pos={with_pos}"
                assert np.all(kept[0, s, h, ref.size:] == -1)


# every tier boundary of the selectors (register tiers, the union's tiers, the re-reading kernel)
TIER_EDGES = [1, 3, 1024, 1025, 4096, 4097, 8192, 8193, 16384, 16385, 32768, 32769, 65536, 65537]


@pytest.mark.parametrize("t_cap", TIER_EDGES)
def test_selectors_at_tier_edges_bit_exact(t_cap):
    # seeded shapes around each boundary: a full head, a ragged one and a short one per sequence,
    # budgets below and above the prompt, ties in the scores; top-k, random and union checked
    # against the oracle on every head
    r = rng(580, t_cap)
    S, L, H, G = 3, 1, 2, int(r.integers(1, 6))
    Ts = [t_cap, int(r.integers(0, t_cap + 1)), min(t_cap, int(r.integers(0, 300)))]
    B = int(r.integers(1, max(2, t_cap // 2) + 1))
    Ps = [int(r.integers(0, min(t_cap, 2 * B) + 1)) for _ in range(S)]
    R = int(r.integers(0, 200))
    pcap = max(Ps)
    name = f"edge-{t_cap}"
    sc = _select_scores(name, "ties", (L, S, H, t_cap))
    hs = _select_scores(name + "-heads", "ties", (L, S, H, G, t_cap))
    Td, Pd = _i32(Ts), _i32(Ps)
    log(f"[edges] t_cap {t_cap}: T {Ts}, P {Ps}, B {B}, R {R}, G {G}")
    kt, nt = kv.kv_select_topk(torch.from_numpy(sc).to(DEV), Td, Pd, B, R, pcap)
    kr, nr = kv.kv_select_random((L, S, H, t_cap), Td, Pd, B, R, pcap, 99, 4)
    ku, nu = kv.kv_select_union(torch.from_numpy(hs).to(DEV), torch.from_numpy(sc).to(DEV), Td, Pd, B, R, pcap)
    kt, kr, ku = kt.cpu().numpy(), kr.cpu().numpy(), ku.cpu().numpy()
    for s in range(S):
        for h in range(H):
            refs = (oracle.select_topk(sc[0, s, h], Ts[s], Ps[s], B, R),
                    oracle.select_random(Ts[s], Ps[s], B, R, None, 99, 4, 0, h, s),
                    oracle.select_union(hs[0, s, h], sc[0, s, h], Ts[s], Ps[s], B, R))
            for what, got, n, ref in zip(("topk", "random", "union"), (kt, kr, ku), (nt, nr, nu), refs):
                assert int(n[s]) == ref.size, f"{name} {what} s{s}"
                assert np.array_equal(got[0, s, h, :ref.size], ref), f"{name} {what} s{s} h{h}"
                assert np.all(got[0, s, h, ref.size:] == -1), f"{name} {what} s{s} h{h} padding"


def test_select_random_layer_chunks_draw_as_one_call():
    # a pass split into layer chunks (each call told its first layer) keeps what one call keeps,
    # and every chunk matches the oracle at the model's layer index
    L, S, H, t_cap = 5, 2, 3, 3000
    Ts, Ps = [3000, 2500], [200, 700]
    B, R, pcap, seed, event = 1000, 64, 700, 0x5EED0000000000AB, 12
    log("[random] layer chunks")
    r = rng(571, t_cap)
    pos = _i32(np.sort(r.integers(0, 2 ** 30, (L, S, H, t_cap)), axis=-1).astype(np.int32))
    whole, nw = kv.kv_select_random((L, S, H, t_cap), _i32(Ts), _i32(Ps), B, R, pcap, seed, event, pos=pos)
    parts = []
    for lo, hi in ((0, 2), (2, 3), (3, 5)):
        k, n = kv.kv_select_random((hi - lo, S, H, t_cap), _i32(Ts), _i32(Ps), B, R, pcap, seed, event,
                                   pos=pos[lo:hi].contiguous(), layer_base=lo)
        assert torch.equal(n, nw)
        parts.append(k)
    assert torch.equal(torch.cat(parts, 0), whole)
    got = parts[2].cpu().numpy()
    p = pos.cpu().numpy()
    for s in range(S):
        for h in range(H):
            ref = oracle.select_random(Ts[s], Ps[s], B, R, p[4, s, h], seed, event, 4, h, s)
            assert np.array_equal(got[1, s, h, :ref.size], ref)


def test_select_random_fresh_per_event_and_head():
    Ts, Ps = [4000], [100]
    a, _ = kv.kv_select_random((1, 1, 2, 4000), _i32(Ts), _i32(Ps), 1000, 32, 100, 9, 1)
    b, _ = kv.kv_select_random((1, 1, 2, 4000), _i32(Ts), _i32(Ps), 1000, 32, 100, 9, 2)
    a, b = a.cpu().numpy(), b.cpu().numpy()
    assert not np.array_equal(a[0, 0, 0], b[0, 0, 0])
    assert not np.array_equal(a[0, 0, 0], a[0, 0, 1])


# ---------------------------------------------------------------- compact ----
COMPACT_CASES = [
    # name, dtype, d, L, S, H, t_cap, n_kept per seq, b_cap, out_cap, with pos_in
    ("bf16-d128", "bf16", 128, 2, 3, 2, 3000, [2048, 3000, 1], 3000, 3000, False),
    ("bf16-d64-pos", "bf16", 64, 2, 2, 3, 2176, [2048, 700], 2100, 2176, True),
    ("bf16-d8", "bf16", 8, 1, 2, 1, 500, [100, 0], 128, 130, True),
    ("bf16-d96", "bf16", 96, 1, 1, 2, 900, [333], 400, 400, False),
    ("fp32-d64", "f32", 64, 1, 1, 1, 512, [128], 128, 128, False),
    ("fp32-d256", "f32", 256, 1, 2, 1, 300, [300, 17], 300, 300, True),
    # an output narrower than n_kept keeps the first out_cap rows
    ("bf16-d128-out-narrower", "bf16", 128, 1, 2, 2, 3000, [2048, 500], 2048, 1000, True),
    ("bf16-d64-out-1", "bf16", 64, 1, 1, 2, 700, [600], 600, 1, False),
]


@pytest.mark.parametrize("case", COMPACT_CASES, ids=[c[0] for c in COMPACT_CASES])
def test_compact_bit_exact(case):
    name, dtype, d, L, S, H, t_cap, nks, b_cap, out_cap, with_pos = case
    log(f"[compact] {name}")
    r = rng(520, d, t_cap)
    Kf = r.standard_normal((L, S, H, t_cap, d)).astype(np.float32)
    Vf = r.standard_normal((L, S, H, t_cap, d)).astype(np.float32)
    Kd, Vd = _to_dev_keys(Kf, dtype), _to_dev_keys(Vf, dtype)
    Kh, Vh = _host_keys(Kd, dtype), _host_keys(Vd, dtype)
    kept = np.full((L, S, H, b_cap), -1, np.int32)
    for l in range(L):
        for s in range(S):
            for h in range(H):
                kept[l, s, h, :nks[s]] = random_kept(l * 100 + s * 10 + h, t_cap, nks[s])
    pos = np.sort(r.integers(0, 10 ** 6, (L, S, H, t_cap)), axis=-1).astype(np.int32) if with_pos else None
    sentinel = -7
    Ko = torch.full((L, S, H, out_cap, d), sentinel, dtype=Kd.dtype, device=DEV)
    Vo = torch.full_like(Ko, sentinel)
    Po = torch.full((L, S, H, out_cap), sentinel, dtype=torch.int32, device=DEV)
    kv.kv_compact(Kd, Vd, _i32(kept), _i32(nks), _i32([t_cap] * S), out_cap,
                  pos=None if pos is None else _i32(pos), K_out=Ko, V_out=Vo, pos_out=Po)
    Ko, Vo, Po = _host_keys(Ko, dtype), _host_keys(Vo, dtype), Po.cpu().numpy()
    sent_k = _host_keys(torch.full((1,), sentinel, dtype=Kd.dtype), dtype)[0]
    for l in range(L):
        for s in range(S):
            for h in range(H):
                n = min(nks[s], out_cap)
                rk, rv, rp = oracle.compact(Kh[l, s, h], Vh[l, s, h], None if pos is None else pos[l, s, h],
                                            kept[l, s, h, :n])
                assert np.array_equal(Ko[l, s, h, :n], rk) and np.array_equal(Vo[l, s, h, :n], rv)
                assert np.array_equal(Po[l, s, h, :n], rp)
                assert np.all(Ko[l, s, h, n:] == sent_k) and np.all(Po[l, s, h, n:] == sentinel)


def test_compact_skips_out_of_range_indices():
    L, S, H, t_cap, d = 1, 1, 1, 64, 64
    Kd = torch.arange(t_cap * d, dtype=torch.float32, device=DEV).reshape(L, S, H, t_cap, d)
    kept = _i32(np.array([[[[0, -1, 63, 64, 1000, 5]]]], np.int32))
    Ko = torch.full((L, S, H, 6, d), -3.0, device=DEV)
    Po = torch.full((L, S, H, 6), -3, dtype=torch.int32, device=DEV)
    kv.kv_compact(Kd, Kd.clone(), kept, _i32([6]), _i32([64]), 6, K_out=Ko, V_out=torch.empty_like(Ko), pos_out=Po)
    Ko, Po = Ko.cpu().numpy(), Po.cpu().numpy()
    assert Po[0, 0, 0].tolist() == [0, -3, 63, -3, -3, 5]
    assert np.all(Ko[0, 0, 0, 1] == -3.0) and np.all(Ko[0, 0, 0, 2] == np.arange(63 * d, 64 * d))


# -------------------------------------------------------------- policy variants ----
@pytest.mark.parametrize("case", SELECT_CASES[:6] + SELECT_CASES[8:12], ids=[c[0] for c in SELECT_CASES[:6] + SELECT_CASES[8:12]])
def test_select_recent_bit_exact(case):
    name, t_cap, Ts, Ps, B, R, _ = case
    log(f"[recent] {name}")
    L, H = 2, 3
    S = len(Ts)
    pcap = max(Ps)
    b_cap = max(B, pcap) + 5
    kept, nk = kv.kv_select_recent((L, S, H, t_cap), _i32(Ts), _i32(Ps), B, R, pcap, b_cap=b_cap)
    kept, nk = kept.cpu().numpy(), nk.cpu().numpy()
    for s in range(S):
        ref = oracle.select_recent(Ts[s], Ps[s], B, R)
        assert nk[s] == ref.size
        for l in range(L):
            for h in range(H):
                assert np.array_equal(kept[l, s, h, :ref.size], ref), f"{name} l{l} s{s} h{h}"
                assert np.all(kept[l, s, h, ref.size:] == -1)


@pytest.mark.parametrize("with_pos", [False, True])
@pytest.mark.parametrize("t_cap", [5000, 70000])
def test_select_random_shared_bit_exact(with_pos, t_cap):
    L, S, H = 3, 2, 4
    Ts, Ps, B, R = [t_cap, 3100], [200, 0], 1500, 64
    seed, event = 0x1234567890ABCDEF, 12
    pos = None
    if with_pos:
        r = rng(511, 0)
        pos = np.sort(r.integers(0, 2 ** 31 - 1, (L, S, H, t_cap)), axis=-1).astype(np.int32)
        pos[:, :, 1] = pos[:, :, 0]           # heads 0 and 1 share positions, the others do not
    kept, nk = kv.kv_select_random_shared((L, S, H, t_cap), _i32(Ts), _i32(Ps), B, R, max(Ps), seed, event,
                                          pos=None if pos is None else _i32(pos))
    kept, nk = kept.cpu().numpy(), nk.cpu().numpy()
    for s in range(S):
        for l in range(L):
            for h in range(H):
                p = None if pos is None else pos[l, s, h]
                ref = oracle.select_random_shared(Ts[s], Ps[s], B, R, p, seed, event, s)
                assert nk[s] == ref.size
                assert np.array_equal(kept[l, s, h, :ref.size], ref), f"shared l{l} s{s} h{h}"
        if pos is None:
            assert np.all(kept[:, s] == kept[0, s, 0][None, None])      # one keep-set for every head
        else:
            assert np.array_equal(kept[:, s, 0], kept[:, s, 1])


HOLE_CASES = [
    # name, dtype, d, L, S, H, t_cap, T per seq, B, R, with pos
    ("holes-bf16-d64-periodic", "bf16", 64, 2, 3, 2, 2176, [2176, 2100, 900], 2048, 128, True),
    ("holes-bf16-d128-deep", "bf16", 128, 1, 2, 2, 9000, [9000, 4000], 3072, 128, True),
    ("holes-fp32-d8-nopos", "f32", 8, 1, 1, 3, 700, [700], 200, 0, False),
    ("holes-bf16-d96", "bf16", 96, 1, 2, 1, 1500, [1500, 1499], 1000, 16, True),
    # kept lists at and past the 4096 entries a workgroup copies to LDS (the longer one searches
    # global memory)
    ("holes-bf16-d64-list4096", "bf16", 64, 1, 1, 2, 6000, [6000], 4096, 128, True),
    ("holes-bf16-d64-list5000", "bf16", 64, 1, 2, 2, 12000, [12000, 7000], 5000, 128, True),
]


@pytest.mark.parametrize("case", HOLE_CASES, ids=[c[0] for c in HOLE_CASES])
def test_compact_inplace_bit_exact(case):
    name, dtype, d, L, S, H, t_cap, Ts, B, R, with_pos = case
    log(f"[holes] {name}")
    r = rng(525, d, t_cap)
    Kf = r.standard_normal((L, S, H, t_cap, d)).astype(np.float32)
    Vf = r.standard_normal((L, S, H, t_cap, d)).astype(np.float32)
    Kd, Vd = _to_dev_keys(Kf, dtype), _to_dev_keys(Vf, dtype)
    Kh, Vh = _host_keys(Kd, dtype), _host_keys(Vd, dtype)
    pos = np.sort(r.integers(0, 10 ** 6, (L, S, H, t_cap)), axis=-1).astype(np.int32) if with_pos else None
    Ps = [min(64, T) for T in Ts]
    kept, nk = kv.kv_select_random((L, S, H, t_cap), _i32(Ts), _i32(Ps), B, R, max(Ps), 5, 3,
                                   pos=None if pos is None else _i32(pos))
    pd = None if pos is None else _i32(pos)
    kv.kv_compact_inplace(Kd, Vd, kept, nk, _i32(Ts), pos=pd)
    Ko, Vo = _host_keys(Kd, dtype), _host_keys(Vd, dtype)
    Po = None if pd is None else pd.cpu().numpy()
    kh, nkh = kept.cpu().numpy(), nk.cpu().numpy()
    moved = 0
    for l in range(L):
        for s in range(S):
            for h in range(H):
                n = int(nkh[s])
                T = Ts[s]
                p = None if pos is None else pos[l, s, h, :T]
                rk, rv, rp, moves = oracle.compact_holes(Kh[l, s, h, :T], Vh[l, s, h, :T], p, kh[l, s, h, :n])
                moved += len(moves)
                assert np.array_equal(Ko[l, s, h, :n], rk) and np.array_equal(Vo[l, s, h, :n], rv), f"{name} {l}{s}{h}"
                if Po is not None:
                    assert np.array_equal(Po[l, s, h, :n], rp)
                    assert np.array_equal(Po[l, s, h, n:], pos[l, s, h, n:])
                assert np.array_equal(Ko[l, s, h, n:], Kh[l, s, h, n:])     # slots >= n untouched
    log(f"[holes] {name}: {moved} rows moved")


UNION_CASES = [
    # name, t_cap, T per seq, P per seq, B, R, G, k_per_head (0: ceil(n_sel / G)), score kind
    ("union-1k-g4", 1000, [1000, 700, 5], [10, 0, 0], 300, 16, 4, 0, "normal"),
    ("union-4k-g8-ties", 4096, [4096, 3000], [100, 2500], 2048, 128, 8, 0, "ties"),
    ("union-8k-g2-long", 8192, [8192, 8000], [512, 0], 2048, 128, 2, 2048, "normal"),
    ("union-16k-g4-specials", 16000, [16000, 12345], [1024, 77], 3072, 128, 4, 0, "specials"),
    ("union-32k-g4", 32768, [32768, 20000], [1024, 4096], 3072, 128, 4, 0, "normal"),
    ("union-32k-g8-k1", 32768, [32768], [512], 2048, 128, 8, 1, "ties"),
    ("union-64k-g2", 65536, [65536, 40000], [1024, 0], 2048, 64, 2, 0, "ties"),
    ("union-g1", 3000, [3000], [100], 500, 10, 1, 0, "normal"),
    ("union-equal", 3000, [3000], [100], 500, 10, 4, 0, "equal"),
    ("union-fits", 3000, [2048, 100], [100, 50], 2048, 128, 4, 0, "normal"),
    ("union-ragged-rows", 2999, [2999, 2500], [7, 0], 700, 9, 3, 0, "specials"),   # t_cap % 4 != 0
    ("union-20k-ragged-rows", 20001, [20001], [300], 2048, 64, 4, 0, "ties"),
    ("union-g64", 4000, [4000, 2500], [100, 0], 1000, 32, 64, 0, "normal"),   # the largest group
    # the prompt is the whole cache (empty evictable range) beside a sequence with none, and a
    # prompt exactly the budget
    ("union-prompt-whole-cache", 3000, [3000, 2600, 1000], [3000, 2600, 0], 2048, 128, 4, 0, "normal"),
    ("union-prompt-equals-budget", 3000, [3000], [2048], 2048, 128, 4, 0, "ties"),
    # past 65536 slots: the re-reading kernel with the union as a bit per slot in LDS
    ("union-stream-70k-g4", 70000, [70000, 65537], [1024, 0], 3072, 128, 4, 0, "normal"),
    ("union-stream-128k-g8-ties", 131072, [131072, 100000], [2048, 10], 4096, 128, 8, 0, "ties"),
    ("union-stream-100k-g2-long", 100000, [100000], [512], 2048, 128, 2, 2048, "normal"),
    ("union-stream-80k-g4-short", 80000, [80000, 3000], [100, 0], 2048, 64, 4, 1, "specials"),
    ("union-stream-70k-crowded", 70000, [70000], [100], 3000, 64, 3, 0, "cluster"),
    ("union-stream-66k-equal", 66000, [66000], [100], 500, 10, 4, 0, "equal"),
    ("union-stream-262k-g4", 262144, [262144, 70001], [1024, 3], 3072, 128, 4, 0, "normal"),
]


@pytest.mark.parametrize("case", UNION_CASES, ids=[c[0] for c in UNION_CASES])
def test_select_union_bit_exact(case):
    name, t_cap, Ts, Ps, B, R, G, k, kind = case
    log(f"[union] {name}")
    L, H = 1, 2
    S = len(Ts)
    hs = _select_scores(name + "-heads", kind, (L, S, H, G, t_cap))
    comb = _select_scores(name + "-combined", kind if kind != "equal" else "normal", (L, S, H, t_cap))
    pcap = max(Ps)
    b_cap = max(B, pcap) + 2
    kept, nk = kv.kv_select_union(torch.from_numpy(hs).to(DEV), torch.from_numpy(comb).to(DEV), _i32(Ts), _i32(Ps),
                                  B, R, pcap, k_per_head=k, b_cap=b_cap)
    kept, nk = kept.cpu().numpy(), nk.cpu().numpy()
    for s in range(S):
        for l in range(L):
            for h in range(H):
                ref = oracle.select_union(hs[l, s, h], comb[l, s, h], Ts[s], Ps[s], B, R, k=k or None)
                assert nk[s] == ref.size
                assert np.array_equal(kept[l, s, h, :ref.size], ref), f"{name} l{l} s{s} h{h}"
                assert np.all(kept[l, s, h, ref.size:] == -1)


def test_calls_run_on_the_current_stream():
    # every call enqueues on torch's current stream: work on a side stream, ordered by events,
    # gives the same bits as on the default stream
    r = rng(570, 0)
    L, S, H, T, d = 2, 2, 3, 3000, 128
    K = _to_dev_keys(r.standard_normal((L, S, H, T, d)).astype(np.float32), "bf16")
    V = K.clone()
    qb = torch.from_numpy(r.standard_normal((L, H, d)).astype(np.float32)).to(DEV)
    Ts, Ps = _i32([T, 2500]), _i32([100, 0])
    args = (1e6, [1, 2, 4, 8])

    def run():
        sc = kv.tri_score(K, qb, Ts, Ts, *args)
        kept, nk = kv.kv_select_topk(sc, Ts, Ps, 1000, 32, 100)
        Ko, Vo, Po = kv.kv_compact(K, V, kept, nk, Ts, 1000)
        return sc, kept, Ko

    ref = run()
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # compare what the calls write: scores of slots < T, the whole kept lists, the first n_kept rows
    for s_, T_ in enumerate((T, 2500)):
        assert torch.equal(ref[0][:, s_, :, :T_].view(torch.int32), got[0][:, s_, :, :T_].view(torch.int32))
    assert torch.equal(ref[1], got[1])
    assert torch.equal(ref[2][..., :1000, :].view(torch.int16), got[2][..., :1000, :].view(torch.int16))


def test_pass_replays_from_a_hip_graph():
    # the calls only launch kernels on the current stream (no allocation, no memset, no sync), so a
    # pass captures into a HIP graph; every replay, with eager work in between that changes the
    # inputs, matches the eager pass on the same inputs bit for bit
    r = rng(571, 0)
    L, S, H, T, d, B = 2, 2, 3, 4000, 128, 1000
    Kf = [r.standard_normal((L, S, H, T, d)).astype(np.float32) for _ in range(3)]
    K = _to_dev_keys(Kf[0], "bf16")
    V = K.clone()
    qb = torch.from_numpy(r.standard_normal((L, H, d)).astype(np.float32)).to(DEV)
    Ts, Ps = _i32([T, 3100]), _i32([100, 0])
    sc = torch.empty((L, S, H, T), device=DEV)
    kept = torch.empty((L, S, H, B), dtype=torch.int32, device=DEV)
    nk = torch.empty((S,), dtype=torch.int32, device=DEV)
    Ko = torch.empty((L, S, H, B, d), dtype=K.dtype, device=DEV)
    Vo = torch.empty_like(Ko)
    Po = torch.empty((L, S, H, B), dtype=torch.int32, device=DEV)
    args = (1e6, [2 ** i for i in range(17)])

    def run():
        kv.tri_score(K, qb, Ts, Ts, *args, out=sc)
        kv.kv_select_topk(sc, Ts, Ps, B, 32, 100, kept=kept, n_kept=nk)
        kv.kv_compact(K, V, kept, nk, Ts, B, K_out=Ko, V_out=Vo, pos_out=Po)

    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()

    def written():
        out = [sc[:, 0].clone(), sc[:, 1, :, :3100].clone(), kept.clone(), nk.clone()]
        n = int(nk[0])
        out += [Ko[:, 0, :, :n].clone(), Vo[:, 0, :, :n].clone(), Po[:, 0, :, :n].clone()]
        n1 = int(nk[1])
        out += [Ko[:, 1, :, :n1].clone(), Po[:, 1, :, :n1].clone()]
        return out

    for rep in range(3):
        K.copy_(_to_dev_keys(Kf[rep], "bf16"))          # eager work between replays
        V.copy_(K.flip(-1))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = written()
        run()
        torch.cuda.synchronize()
        ref = written()
        for a, b in zip(got, ref):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), f"replay {rep}"


def test_next_row_calls_replay_from_a_hip_graph():
    # the next rows' calls capture too: grouped-query scores (caller workspace), union, random,
    # recency and in-place compaction; each replay matches the eager calls on changed inputs
    r = rng(572, 0)
    L, S, H, T, d, G, B = 1, 2, 2, 3000, 64, 4, 800
    Kf = [r.standard_normal((L, S, H, T, d)).astype(np.float32) for _ in range(3)]
    K = _to_dev_keys(Kf[0], "bf16")
    nu = torch.from_numpy(r.standard_normal((L, H, G, d)).astype(np.float32)).to(DEV)
    Ts, Ps = _i32([T, 2100]), _i32([64, 0])
    z = torch.empty((L, S, H, T), device=DEV)
    hs = torch.empty((L, S, H, G, T), device=DEV)
    ws = torch.empty((kv.gqa_workspace_bytes(L, S, H, T, d, K.dtype, G),), dtype=torch.uint8, device=DEV)
    outs = {k: (torch.empty((L, S, H, B), dtype=torch.int32, device=DEV), torch.empty((S,), dtype=torch.int32, device=DEV))
            for k in ("union", "random", "recent")}
    Kc, Vc, Pc = K.clone(), K.clone(), torch.arange(T, dtype=torch.int32, device=DEV).expand(L, S, H, T).contiguous()
    args = (1e4, [1, 2, 4, 8, 16])

    def run():
        kv.tri_score_gqa(K, nu, Ts, Ts, *args, out=z, head_out=hs, workspace=ws)
        kv.kv_select_union(hs, z, Ts, Ps, B, 16, 64, kept=outs["union"][0], n_kept=outs["union"][1])
        kv.kv_select_random((L, S, H, T), Ts, Ps, B, 16, 64, 5, 3, kept=outs["random"][0], n_kept=outs["random"][1])
        kv.kv_select_recent((L, S, H, T), Ts, Ps, B, 16, 64, kept=outs["recent"][0], n_kept=outs["recent"][1])
        kv.kv_compact_inplace(Kc, Vc, outs["union"][0], outs["union"][1], Ts, pos=Pc)

    def reset(rep):
        K.copy_(_to_dev_keys(Kf[rep], "bf16"))
        Kc.copy_(K)
        Vc.copy_(K.flip(-1))
        Pc.copy_(torch.arange(T, dtype=torch.int32, device=DEV).expand(L, S, H, T))

    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()

    def written():
        got = [z[:, 0].clone(), z[:, 1, :, :2100].clone(), hs[:, 0].clone(), hs[:, 1, :, :, :2100].clone()]
        for k in ("union", "random", "recent"):
            got += [outs[k][0].clone(), outs[k][1].clone()]
        got += [Kc.clone(), Vc.clone(), Pc.clone()]
        return got

    for rep in range(3):
        reset(rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = written()
        reset(rep)
        run()
        torch.cuda.synchronize()
        ref = written()
        for i, (a, b) in enumerate(zip(got, ref)):
            bits = (lambda x: x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32))
            assert torch.equal(bits(a), bits(b)), f"replay {rep}, output {i}"


def test_audit_accepts_every_selector_and_flags_broken_lists():
    L, S, H, t_cap = 2, 3, 2, 5000
    Ts, Ps, B, R = [5000, 1800, 4000], [100, 0, 3900], 2000, 64
    pcap = max(Ps)
    sc = torch.from_numpy(random_scores(77, (L, S, H, t_cap), ties=0.2)).to(DEV)
    hs = torch.from_numpy(random_scores(78, (L, S, H, 3, t_cap))).to(DEV)
    Td, Pd = _i32(Ts), _i32(Ps)
    lists = {
        "topk": kv.kv_select_topk(sc, Td, Pd, B, R, pcap),
        "random": kv.kv_select_random((L, S, H, t_cap), Td, Pd, B, R, pcap, 5, 1),
        "shared": kv.kv_select_random_shared((L, S, H, t_cap), Td, Pd, B, R, pcap, 5, 1),
        "recent": kv.kv_select_recent((L, S, H, t_cap), Td, Pd, B, R, pcap),
        "union": kv.kv_select_union(hs, sc, Td, Pd, B, R, pcap),
    }
    for name, (kept, nk) in lists.items():
        bad = kv.kv_audit_kept(kept, nk, Td, Pd, B, R, pcap, t_cap)
        assert int(bad.abs().sum()) == 0, name
    kept, nk = lists["topk"]
    k2 = kept.clone()
    k2[0, 0, 0, 500], k2[0, 0, 0, 501] = kept[0, 0, 0, 501], kept[0, 0, 0, 500]     # order broken
    k2[1, 2, 1, 7] = 3999                                                             # prompt slot replaced
    k2[0, 1, 1, nk[1].item()] = 0                                                    # padding overwritten
    bad = kv.kv_audit_kept(k2, nk, Td, Pd, B, R, pcap, t_cap).cpu().numpy()
    assert bad[0, 0, 0] >= 1 and bad[1, 2, 1] >= 1 and bad[0, 1, 1] == 1
    assert bad.sum() == bad[0, 0, 0] + bad[1, 2, 1] + bad[0, 1, 1]
    nk2 = nk.clone()
    nk2[2] += 1
    bad = kv.kv_audit_kept(kept, nk2, Td, Pd, B, R, pcap, t_cap).cpu().numpy()
    assert np.all(bad[:, 2] == 1) and bad[:, :2].sum() == 0


def test_every_other_entry_point_is_deterministic():
    # each call run twice on the same inputs gives the same bits (score, GQA and the scored pass are
    # covered by their own tests): rotated keys dense and paged, grouped-query scores over rotated
    # keys, random / shared / recency / union selection, the audit, both compactions
    log("[determinism] every other entry point")
    r = rng(777, 1)
    L, S, H, T, d, G, B, R = 2, 3, 2, 3008, 128, 4, 700, 64
    Ts = _i32([3000, 2500, 1700])
    Ps = _i32([100, 800, 10])
    tcur = _i32([3004, 2600, 1800])
    D = [2 ** i for i in range(17)]
    K = _to_dev_keys((r.standard_normal((L, 1, H, 1, d)) + 0.3 * r.standard_normal((L, S, H, T, d))).astype(np.float32),
                     "bf16")
    V = _to_dev_keys(r.standard_normal((L, S, H, T, d)).astype(np.float32), "bf16")
    pos = torch.from_numpy(np.sort(r.integers(0, 10 ** 6, (L, S, H, T)), axis=-1).astype(np.int32)).to(DEV)
    qb = torch.from_numpy(r.standard_normal((L, H, d)).astype(np.float32)).to(DEV)
    nu = torch.from_numpy(r.standard_normal((L, H, G, d)).astype(np.float32)).to(DEV)
    bs = 16
    bps = T // bs
    pool = K.view(L, S * bps, bs, H, d)
    table = _i32(r.permutation(S * bps).reshape(S, bps))
    pc = int(Ps.max())

    def same(a, b, what):
        a = a if isinstance(a, tuple) else (a,)
        b = b if isinstance(b, tuple) else (b,)
        for x, y in zip(a, b):
            assert torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x,
                               y.view(torch.int32) if y.dtype == torch.float32 else y), what

    Tl = Ts.cpu().tolist()

    def written(x):
        # score outputs hold nothing at or past a sequence's length: compare the written slots
        y = x.clone()
        for si, t in enumerate(Tl):
            y[:, si, ..., t:] = 0
        return y

    calls = {
        "rotated dense": lambda: kv.tri_score_rotated(K, qb, tcur, Ts, 1e6, D),
        "rotated paged": lambda: kv.tri_score_rotated(pool, qb, tcur, Ts, 1e6, D, block_table=table),
        "gqa rotated paged": lambda: kv.tri_score_gqa_rotated(pool, nu, tcur, Ts, 1e6, D, block_table=table),
        "random": lambda: kv.kv_select_random((L, S, H, T), Ts, Ps, B, R, pc, 99, 4, pos=pos),
        "random shared": lambda: kv.kv_select_random_shared((L, S, H, T), Ts, Ps, B, R, pc, 99, 4),
        "recent": lambda: kv.kv_select_recent((L, S, H, T), Ts, Ps, B, R, pc),
    }
    out = {}
    for name, fn in calls.items():
        a, b = fn(), fn()
        if name.startswith(("rotated", "gqa")):
            a = tuple(written(x) for x in a) if isinstance(a, tuple) else written(a)
            b = tuple(written(x) for x in b) if isinstance(b, tuple) else written(b)
        same(a, b, name)
        out[name] = a
    zmax, head = out["gqa rotated paged"]
    u1 = kv.kv_select_union(head, zmax, Ts, Ps, B, R, pc)
    same(u1, kv.kv_select_union(head, zmax, Ts, Ps, B, R, pc), "union")
    kept, nk = out["random"]
    a1 = kv.kv_audit_kept(kept, nk, Ts, Ps, B, R, pc, T)
    same(a1, kv.kv_audit_kept(kept, nk, Ts, Ps, B, R, pc, T), "audit")
    assert int(a1.sum()) == 0
    oc = max(B, pc)                 # a prompt longer than the budget is kept whole
    outs = []
    for _ in range(2):              # rows past n_kept are not written: start both from zeros
        Ko = torch.zeros((L, S, H, oc, d), dtype=K.dtype, device=DEV)
        Vo, Po = torch.zeros_like(Ko), torch.zeros((L, S, H, oc), dtype=torch.int32, device=DEV)
        kv.kv_compact(K, V, kept, nk, Ts, oc, pos=pos, K_out=Ko, V_out=Vo, pos_out=Po)
        outs.append((Ko.view(torch.int16), Vo.view(torch.int16), Po))
    same(outs[0], outs[1], "compact")
    Ka, Va, Pa = K.clone(), V.clone(), pos.clone()
    Kb, Vb, Pb = K.clone(), V.clone(), pos.clone()
    kv.kv_compact_inplace(Ka, Va, kept, nk, Ts, pos=Pa)
    kv.kv_compact_inplace(Kb, Vb, kept, nk, Ts, pos=Pb)
    same((Ka.view(torch.int16), Va.view(torch.int16), Pa), (Kb.view(torch.int16), Vb.view(torch.int16), Pb), "in place")
    log("[determinism] all bit-identical")


@pytest.mark.parametrize("sweep", range(16))
def test_selectors_random_sweep(sweep):
    # random ragged batches (lengths, prompts, budget, window and cache capacity drawn per sweep,
    # crossing the register tiers): top-k on scores with ties and special values, random with and
    # without positions, recency and union, every head bit-exact against the oracle
    r = rng(4242, sweep)
    t_cap = int(r.choice([37, 300, 1029, 4096, 9000, 20001, 32768, 40000]))
    S, H, G = int(r.integers(1, 9)), 2, int(r.integers(1, 5))
    B = int(r.integers(1, max(2, t_cap)))
    R = int(r.integers(0, 200))
    Ts = r.integers(0, t_cap + 1, S).astype(np.int32)
    Ts[0] = t_cap
    Ps = np.minimum(r.integers(0, max(1, t_cap // 2), S), Ts).astype(np.int32)
    pc = int(Ps.max())
    log(f"[sweep {sweep}] t_cap={t_cap} S={S} B={B} R={R} G={G} T={Ts.tolist()} P={Ps.tolist()}")
    sc = random_scores(700 + sweep, (1, S, H, t_cap), ties=0.2, specials=True)
    hs = random_scores(800 + sweep, (1, S, H, G, t_cap), ties=0.3, specials=sweep % 2 == 0)
    pos = np.sort(r.integers(0, 2 ** 31 - 1, (1, S, H, t_cap)), axis=-1).astype(np.int32)
    seed, event = int(r.integers(0, 2 ** 63)), int(r.integers(0, 1000))
    Tt, Pt = _i32(Ts), _i32(Ps)
    got = {
        "topk": kv.kv_select_topk(torch.from_numpy(sc).to(DEV), Tt, Pt, B, R, pc),
        "random": kv.kv_select_random((1, S, H, t_cap), Tt, Pt, B, R, pc, seed, event),
        "random-pos": kv.kv_select_random((1, S, H, t_cap), Tt, Pt, B, R, pc, seed, event, pos=_i32(pos)),
        "recent": kv.kv_select_recent((1, S, H, t_cap), Tt, Pt, B, R, pc),
        "union": kv.kv_select_union(torch.from_numpy(hs).to(DEV), torch.from_numpy(sc).to(DEV), Tt, Pt, B, R, pc),
    }
    got = {k: (v[0].cpu().numpy(), v[1].cpu().numpy()) for k, v in got.items()}
    for s in range(S):
        T, P = int(Ts[s]), int(Ps[s])
        for h in range(H):
            want = {
                "topk": oracle.select_topk(sc[0, s, h, :T], T, P, B, R),
                "random": oracle.select_random(T, P, B, R, None, seed, event, 0, h, s),
                "random-pos": oracle.select_random(T, P, B, R, pos[0, s, h, :T], seed, event, 0, h, s),
                "recent": oracle.select_recent(T, P, B, R),
                "union": oracle.select_union(hs[0, s, h, :, :T], sc[0, s, h, :T], T, P, B, R),
            }
            for name, ref in want.items():
                kept, nk = got[name]
                assert int(nk[s]) == ref.size, (name, s, h)
                assert np.array_equal(kept[0, s, h, :ref.size], ref), (name, s, h)
                assert np.all(kept[0, s, h, ref.size:] == -1), (name, s, h)
    log(f"[sweep {sweep}] all heads bit-exact")


@pytest.mark.parametrize("sweep", range(16))
def test_scores_random_sweep(sweep):
    # random shapes within each call's limits: dtype, head_dim (every multiple of a 16-byte piece),
    # lengths, theta, offsets, explicit positions, the norm term, pairing and group size; every head
    # of tri_score, tri_score_rotated, tri_score_gqa (scores and z) and tri_score_gqa_rotated
    # against the oracle
    r = rng(4343, sweep)
    dtype = "bf16" if sweep % 3 else "f32"
    step = 8 if dtype == "bf16" else 4
    d = int(r.integers(1, (256 if sweep % 2 else 128) // step + 1)) * step   # half the draws at most 128
    S, H = int(r.integers(1, 4)), int(r.integers(1, 3))
    t_cap = int(r.integers(1, 2500))
    Ts = r.integers(0, t_cap + 1, S).astype(np.int32)
    Ts[0] = t_cap
    t_cur = (Ts + r.integers(0, 50, S)).astype(np.int32)
    theta = float(r.choice([1e4, 5e5, 1e6]))
    D = sorted(set(r.integers(0, 65537, int(r.integers(1, 18))).tolist()))
    with_pos, norm = bool(r.integers(0, 2)), bool(r.integers(0, 2))
    style = "half" if r.integers(0, 2) else "interleaved"
    pc = d * (2 if dtype == "bf16" else 4) // 16
    if pc < 2 or pc & (pc - 1):
        style = "interleaved"      # half-split rows need a power-of-two number (>= 2) of pieces
    G = int(r.integers(1, 9))
    log(f"[score sweep {sweep}] {dtype} d={d} S={S} H={H} t_cap={t_cap} T={Ts.tolist()} |D|={len(D)} "
        f"pos={with_pos} norm={norm} style={style} G={G}")
    K = (r.standard_normal((1, 1, H, 1, d)) + 0.3 * r.standard_normal((1, S, H, t_cap, d))).astype(np.float32)
    Kd = _to_dev_keys(K, dtype)
    Kh = keys_f64(_host_keys(Kd, dtype), dtype)
    pos = np.sort(r.integers(0, 2 ** 20, (1, S, H, t_cap)), axis=-1).astype(np.int32) if with_pos else None
    pos_d = None if pos is None else _i32(pos)
    qb = r.standard_normal((1, H, d)).astype(np.float32)
    nu = r.standard_normal((1, H, G, d)).astype(np.float32)

    def magnitudes(c, pairing):
        re, im = oracle.band_slices(d, pairing)
        return (np.hypot(c[..., re], c[..., im]) / r.uniform(0.6, 1.0, c.shape[:-1] + (d // 2,))).astype(np.float32)

    qabs_i = magnitudes(qb, "interleaved") if norm else None
    qabs_s = magnitudes(qb, style) if norm else None
    tc, Tt = _i32(t_cur), _i32(Ts)
    dev = lambda a: None if a is None else torch.from_numpy(a).to(DEV)
    got_pre = kv.tri_score(Kd, dev(qb), tc, Tt, theta, D, pos=pos_d, qabs=dev(qabs_i)).cpu().numpy()
    pieces = d * (2 if dtype == "bf16" else 4) // 16
    # half-split rows: a power-of-two number (>= 2) of 16-byte pieces, so a band's halves sit in
    # lanes g and g ^ (lanes / 2)
    half_ok = style == "interleaved" or (pieces >= 2 and pieces & (pieces - 1) == 0)
    got_rot = kv.tri_score_rotated(Kd, dev(qb), tc, Tt, theta, D, rope_style=style,
                                   qabs=dev(qabs_s)).cpu().numpy() if half_ok else None
    gqa_ok = d <= (256 if dtype == "bf16" else 128)
    qabs_g = magnitudes(nu, "interleaved") if norm else None
    got_gqa = kv.tri_score_gqa(Kd, dev(nu), tc, Tt, theta, D, pos=pos_d, qabs=dev(qabs_g)) if gqa_ok else None
    lpk = 1 << (pieces - 1).bit_length()
    grot_ok = lpk <= 16 and (style == "interleaved" or (lpk == pieces and lpk >= 2))
    qabs_gs = magnitudes(nu, style) if norm else None
    got_grot = kv.tri_score_gqa_rotated(Kd, dev(nu), tc, Tt, theta, D, rope_style=style,
                                        qabs=dev(qabs_gs)) if grot_ok else None
    worst = 0.0
    for s in range(S):
        T, t = int(Ts[s]), int(t_cur[s])
        for h in range(H):
            kf, ps = Kh[0, s, h, :T], None if pos is None else pos[0, s, h, :T]
            ref = oracle.score_full(kf, ps, qb[0, h], qabs_i[0, h], t, theta, D) if norm else \
                oracle.score_literal(kf, ps, qb[0, h], t, theta, D)
            worst = max(worst, assert_scores(got_pre[0, s, h, :T], ref, f"tri_score {s} {h}"))
            if got_rot is not None:
                ref = oracle.score_rotated(kf, qb[0, h], t, theta, D, style, None if qabs_s is None else qabs_s[0, h])
                worst = max(worst, assert_scores(got_rot[0, s, h, :T], ref, f"rotated {s} {h}"))
            if got_gqa is not None:
                z, per = oracle.score_gqa(kf, ps, nu[0, h], t, theta, D, None if qabs_g is None else qabs_g[0, h])
                zg, hg = got_gqa[0][0, s, h, :T].cpu().numpy(), got_gqa[1][0, s, h, :, :T].cpu().numpy()
                for g in range(G):
                    worst = max(worst, assert_scores(hg[g], per[g], f"gqa {s} {h} g{g}"))
                assert_z(zg, z, f"gqa z {s} {h}")
            if got_grot is not None:
                z, per = oracle.score_gqa_rotated(kf, nu[0, h], t, theta, D, style,
                                                  None if qabs_gs is None else qabs_gs[0, h])
                zg, hg = got_grot[0][0, s, h, :T].cpu().numpy(), got_grot[1][0, s, h, :, :T].cpu().numpy()
                for g in range(G):
                    worst = max(worst, assert_scores(hg[g], per[g], f"gqa rotated {s} {h} g{g}"))
                assert_z(zg, z, f"gqa rotated z {s} {h}")
    log(f"[score sweep {sweep}] rotated={got_rot is not None} gqa={got_gqa is not None} "
        f"gqa_rotated={got_grot is not None}: worst scaled error {worst:.2e}")


@pytest.mark.parametrize("sweep", range(12))
def test_compaction_random_sweep(sweep):
    # random row widths (every multiple of a 16-byte piece up to 256 elements), dtypes, lengths,
    # budgets and positions: the gather and in-place hole filling bit-exact against the oracle, on
    # kept lists from random selection
    r = rng(4444, sweep)
    dtype = "bf16" if sweep % 2 else "f32"
    step = 8 if dtype == "bf16" else 4
    d = int(r.integers(1, 256 // step + 1)) * step
    S, H = int(r.integers(1, 4)), int(r.integers(1, 3))
    t_cap = int(r.integers(1, 3000))
    Ts = r.integers(0, t_cap + 1, S).astype(np.int32)
    Ts[0] = t_cap
    Ps = np.minimum(r.integers(0, max(1, t_cap // 3), S), Ts).astype(np.int32)
    B, R = int(r.integers(1, max(2, t_cap))), int(r.integers(0, 100))
    with_pos = bool(r.integers(0, 2))
    log(f"[compact sweep {sweep}] {dtype} d={d} S={S} H={H} t_cap={t_cap} T={Ts.tolist()} P={Ps.tolist()} "
        f"B={B} R={R} pos={with_pos}")
    Kf = r.standard_normal((1, S, H, t_cap, d)).astype(np.float32)
    Vf = r.standard_normal((1, S, H, t_cap, d)).astype(np.float32)
    Kd, Vd = _to_dev_keys(Kf, dtype), _to_dev_keys(Vf, dtype)
    Kh, Vh = _host_keys(Kd, dtype), _host_keys(Vd, dtype)
    pos = np.sort(r.integers(0, 2 ** 30, (1, S, H, t_cap)), axis=-1).astype(np.int32) if with_pos else None
    pd = None if pos is None else _i32(pos)
    kept, nk = kv.kv_select_random((1, S, H, t_cap), _i32(Ts), _i32(Ps), B, R, int(Ps.max()), 17 + sweep, 2)
    oc = max(B, int(Ps.max()), 1)
    Ko, Vo, Po = kv.kv_compact(Kd, Vd, kept, nk, _i32(Ts), oc, pos=pd)
    Ko, Vo, Po = _host_keys(Ko, dtype), _host_keys(Vo, dtype), Po.cpu().numpy()
    kv.kv_compact_inplace(Kd, Vd, kept, nk, _i32(Ts), pos=pd)
    Ki, Vi = _host_keys(Kd, dtype), _host_keys(Vd, dtype)
    Pi = None if pd is None else pd.cpu().numpy()
    kh, nkh = kept.cpu().numpy(), nk.cpu().numpy()
    for s in range(S):
        n, T = int(nkh[s]), int(Ts[s])
        for h in range(H):
            ks = kh[0, s, h, :n]
            p = None if pos is None else pos[0, s, h, :T]
            rk, rv, rp = oracle.compact(Kh[0, s, h, :T], Vh[0, s, h, :T], p, ks)
            assert np.array_equal(Ko[0, s, h, :n], rk) and np.array_equal(Vo[0, s, h, :n], rv), ("gather", s, h)
            assert np.array_equal(Po[0, s, h, :n], rp), ("gather positions", s, h)
            hk, hv, hp, _ = oracle.compact_holes(Kh[0, s, h, :T], Vh[0, s, h, :T], p, ks)
            assert np.array_equal(Ki[0, s, h, :n], hk) and np.array_equal(Vi[0, s, h, :n], hv), ("in place", s, h)
            assert np.array_equal(Ki[0, s, h, n:], Kh[0, s, h, n:]), ("in place tail", s, h)
            if Pi is not None:
                assert np.array_equal(Pi[0, s, h, :n], hp), ("in place positions", s, h)
    log(f"[compact sweep {sweep}] bit-exact")


@pytest.mark.gpu
@pytest.mark.parametrize("with_stores", [True, False])
def test_stream_ceiling_reads_every_byte_once(with_stores):
    """The measurement aid's output is a fixed XOR of what it read: wave w covers bytes
    [32 KB w, 32 KB (w+1)), lane l of batch b takes the 16-byte pieces at 16 KB b + 1 KB t + 16 l
    (t = 0..15). With stores each (wave, batch, lane) value lands in word 128 w + 64 b + l; without,
    word w holds the XOR over all of them. A missed or doubled piece changes the result."""
    n_bytes = 3 * 131072
    words = rng(41).integers(0, 2**32, size=n_bytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to(DEV)
    per = words.reshape(n_bytes // 32768, 2, 16, 64, 4)
    lane_x = np.bitwise_xor.reduce(np.bitwise_xor.reduce(per, axis=4), axis=2)   # [waves, 2, 64]
    if with_stores:
        want = lane_x.reshape(-1)
    else:
        want = np.bitwise_xor.reduce(lane_x.reshape(lane_x.shape[0], -1), axis=1)
    out = torch.full((want.size + 8,), -7, dtype=torch.int32, device=DEV)
    kv.stream_ceiling(buf, out, with_stores)
    got = out.cpu().numpy().view(np.uint32)
    assert np.array_equal(got[:want.size], want)
    assert (got[want.size:] == np.uint32(2**32 - 7)).all()   # nothing past the output

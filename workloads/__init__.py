"""Seeded synthetic inputs for the KV-eviction hot path.

This module is shared by the HIP path's tests/bench and by the CPU oracle's
tests. It holds random draws, shapes and per-sequence lengths only: no
scoring, selection, random-eviction or compaction arithmetic lives here.

The five workloads follow the shapes the pages measure on (32K-token
reasoning generations, budgets of 2048/3072 entries per KV head, ~1k-token
prompts, a 128-token pruning window and 17 geometric future offsets); the
pages' evaluation sets are not available and are not reproduced -- these
draws stand in for them.

Value recipes (readings of under-specified workload text):
  * keys are concentrated pre-RoPE vectors: k = mu + noise * N(0, 1) with a
    per-(layer, KV head) centre mu ~ N(0, 1)^d;
  * the query centre q_bar is either nu + 0.1 * N(0, 1) (tiny and full-pass
    workloads) or the fp32 mean of G per-query-head centres nu_g ~ N(0, 1)^d
    (GQA workloads);
  * values are N(0, 1);
  * bf16 tensors are produced from fp32 draws by round-to-nearest-even.

Small arrays (centres, lengths) always come from NumPy PCG64 streams keyed by
``SeedSequence([SEED_ROOT, workload, layer/part, kind])``. Bulk key/value noise
for the multi-GB workloads is drawn on the device with ``torch.Generator``
seeded from the same key, so that the 39 GB full-pass cache is generated in
seconds; the parity tests copy the slices they check back to the host.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence, Tuple

import numpy as np

SEED_ROOT = 20261202

# kinds of draws (the last SeedSequence word)
K_MU, K_NU, K_KEYNOISE, K_QNOISE, K_VAL, K_LEN, K_DRIFT, K_NEWKEY, K_NEWVAL, K_QABS = range(10)


def rng(*ids: int) -> np.random.Generator:
    """A NumPy PCG64 generator for the stream keyed by ``ids``."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, *ids])))


def torch_seed(*ids: int) -> int:
    """A 63-bit torch seed derived from the same key space as :func:`rng`."""
    st = np.random.SeedSequence([SEED_ROOT, *ids]).generate_state(1, np.uint64)[0]
    return int(st) & ((1 << 63) - 1)


# ----------------------------------------------------------------------------
# bf16 helpers (bit-level; no arithmetic of the method)
# ----------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = ((b >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    return ((b + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# workload descriptions
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    """Shapes, policy and per-sequence lengths of one synthetic workload.

    Cache layout is ``[n_layers, n_seq, n_kv_heads, t_cap, head_dim]`` with
    slot ``j`` of a head holding the token at position ``j`` unless an
    explicit position array is supplied.
    """

    name: str
    wid: int
    n_layers: int
    n_seq: int
    n_kv_heads: int
    group: int                 # query heads per KV head
    head_dim: int
    dtype: str                 # "f32" | "bf16"
    t_cap: int
    seq_len: np.ndarray        # int32 [n_seq]
    prompt_len: np.ndarray     # int32 [n_seq]
    t_cur: np.ndarray          # int32 [n_seq], current (next) position
    budget: int
    recent: int
    theta: float
    deltas: Tuple[int, ...]
    key_noise: float
    q_mode: str                # "nu+noise" | "group-mean"
    q_noise: float = 0.1
    out_cap: int = 0
    drift: float = 0.0         # centre drift per 1000 positions (periodic workload)
    new_per_event: int = 0     # tokens appended between events (periodic workload)
    n_events: int = 0
    seed_random: int = 0       # Philox seed for the random selector
    note: str = ""

    @property
    def n_bands(self) -> int:
        return self.head_dim // 2

    @property
    def n_heads_total(self) -> int:
        return self.n_layers * self.n_seq * self.n_kv_heads

    @property
    def entries(self) -> int:
        """KV entries (layer, seq, KV head, slot) in one pass."""
        return int(self.n_layers * self.n_kv_heads * np.sum(self.seq_len.astype(np.int64)))

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def prompt_cap(self) -> int:
        return int(self.prompt_len.max()) if self.n_seq else 0

    def b_cap(self) -> int:
        return max(self.budget, self.prompt_cap())


GEOMETRIC_17 = tuple(2 ** i for i in range(17))


def workload(wid: int, **over) -> Workload:
    """The five synthetic workloads (``wid`` 1..5); ``over`` rescales for tests."""
    if wid == 1:
        T = over.pop("T", 512)
        w = Workload(
            name="tiny-fp32-d64", wid=1, n_layers=1, n_seq=1, n_kv_heads=1, group=1,
            head_dim=64, dtype="f32", t_cap=T,
            seq_len=np.array([T], np.int32), prompt_len=np.array([64], np.int32),
            t_cur=np.array([T], np.int32), budget=128, recent=16, theta=1e4,
            deltas=tuple(2 ** i for i in range(7)), key_noise=0.3, q_mode="nu+noise",
            note="single head, T=512, P=64, R=16, B=128, t=512",
        )
    elif wid == 2:
        T = over.pop("T", 32768)
        w = Workload(
            name="qwen3-8b-layer-32k", wid=2, n_layers=1, n_seq=1, n_kv_heads=8, group=4,
            head_dim=128, dtype="bf16", t_cap=T,
            seq_len=np.array([T], np.int32), prompt_len=np.array([min(512, T)], np.int32),
            t_cur=np.array([T], np.int32), budget=2048, recent=128, theta=1e6,
            deltas=GEOMETRIC_17, key_noise=0.25, q_mode="group-mean",
            note="one Qwen3-8B-shaped layer, 8 KV heads (GQA 4), T=32768",
        )
    elif wid == 3:
        L = over.pop("L", 36)
        S = over.pop("S", 8)
        T = over.pop("T", 32768)
        w = Workload(
            name="qwen3-8b-full-pass-32k", wid=3, n_layers=L, n_seq=S, n_kv_heads=8, group=4,
            head_dim=128, dtype="bf16", t_cap=T,
            seq_len=np.full(S, T, np.int32), prompt_len=np.full(S, min(1024, T), np.int32),
            t_cur=np.full(S, T, np.int32), budget=3072, recent=128, theta=1e6,
            deltas=GEOMETRIC_17, key_noise=0.3, q_mode="nu+noise",
            note="36 layers x 8 seqs x 8 KV heads, T=32768, P=1024, B=3072",
        )
    elif wid == 4:
        L = over.pop("L", 24)
        S = over.pop("S", 64)
        r = rng(4, 0, K_LEN)
        P = r.integers(256, 2048, size=S, endpoint=True).astype(np.int32)
        B, NEW = 2048, 128
        w = Workload(
            name="gpt-oss-20b-periodic", wid=4, n_layers=L, n_seq=S, n_kv_heads=8, group=8,
            head_dim=64, dtype="bf16", t_cap=B + NEW,
            seq_len=P.copy(), prompt_len=P, t_cur=P.copy(), budget=B, recent=128, theta=1e4,
            deltas=GEOMETRIC_17, key_noise=0.3, q_mode="group-mean", drift=0.01,
            new_per_event=NEW, n_events=over.pop("n_events", 256),
            seed_random=0x5EED000000000004,
            note="24 layers x 64 seqs x 8 KV heads, d=64, B=2048 + 128 per event",
        )
    elif wid == 5:
        S = over.pop("S", 128)
        Tmin, Tmax = over.pop("T_range", (4096, 32768))
        Pmin, Pmax = over.pop("P_range", (128, 4096))
        r = rng(5, 0, K_LEN)
        T = r.integers(Tmin, Tmax, size=S, endpoint=True).astype(np.int32)
        P = r.integers(Pmin, Pmax, size=S, endpoint=True).astype(np.int32)
        P = np.minimum(P, T)
        w = Workload(
            name="ragged-128-scored-vs-random", wid=5, n_layers=1, n_seq=S, n_kv_heads=8,
            group=4, head_dim=128, dtype="bf16", t_cap=int(Tmax),
            seq_len=T, prompt_len=P, t_cur=T.copy(), budget=2048, recent=128, theta=1e6,
            deltas=GEOMETRIC_17, key_noise=0.25, q_mode="group-mean",
            seed_random=0x5EED000000000005,
            note="128 ragged seqs, T~U[4096,32768], P~U[128,4096], B=2048",
        )
    else:
        raise ValueError(f"unknown workload {wid}")
    for k, v in over.items():
        setattr(w, k, v)
    if not w.out_cap:
        w.out_cap = w.b_cap()
    return w


# ----------------------------------------------------------------------------
# small per-(layer, head) parameters: NumPy
# ----------------------------------------------------------------------------
def centres(w: Workload) -> Tuple[np.ndarray, np.ndarray, Optional[np.ndarray]]:
    """Key centres mu [L,H,d], query centres q_bar [L,H,d] (fp32), drift dirs or None."""
    L, H, d = w.n_layers, w.n_kv_heads, w.head_dim
    mu = np.empty((L, H, d), np.float32)
    qb = np.empty((L, H, d), np.float32)
    dr = np.empty((L, H, d), np.float32) if w.drift else None
    for l in range(L):
        mu[l] = rng(w.wid, l, K_MU).standard_normal((H, d)).astype(np.float32)
        if w.q_mode == "nu+noise":
            nu = rng(w.wid, l, K_NU).standard_normal((H, d))
            qb[l] = (nu + w.q_noise * rng(w.wid, l, K_QNOISE).standard_normal((H, d))).astype(np.float32)
        else:
            nu = rng(w.wid, l, K_NU).standard_normal((H, w.group, d)).astype(np.float32)
            qb[l] = nu.mean(axis=1, dtype=np.float64).astype(np.float32)
        if dr is not None:
            dr[l] = rng(w.wid, l, K_DRIFT).standard_normal((H, d)).astype(np.float32)
    return mu, qb, dr


def query_head_centres(w: Workload) -> np.ndarray:
    """Per-query-head centres nu_g, fp32 [L,H,G,d] (the draws whose mean is q_bar in GQA workloads)."""
    if w.q_mode != "group-mean":
        raise ValueError("per-query-head centres exist only for group-mean workloads")
    L, H, d = w.n_layers, w.n_kv_heads, w.head_dim
    return np.stack([rng(w.wid, l, K_NU).standard_normal((H, w.group, d)).astype(np.float32) for l in range(L)])


def query_head_magnitudes(w: Workload, nu: np.ndarray) -> np.ndarray:
    """E|q_f| = |nu_{g,f}| / R_{g,f} per query head, fp32 [L,H,G,d/2]; R ~ U(0.85, 1.0)."""
    L, H, G, F = w.n_layers, w.n_kv_heads, w.group, w.n_bands
    q = np.asarray(nu, np.float64)
    centre = np.abs(q[..., 0::2] + 1j * q[..., 1::2])
    R = np.stack([rng(w.wid, l, K_QABS, 1).uniform(0.85, 1.0, (H, G, F)) for l in range(L)])
    return (centre / R).astype(np.float32)


def query_magnitudes(w: Workload, qbar: np.ndarray) -> np.ndarray:
    """Mean query magnitude per band, E|q_f| = |q_bar_f| / R_f, fp32 [L,H,d/2].

    The mean resultant length R_f is drawn U(0.85, 1.0) per (layer, KV head, band): most
    heads are highly concentrated, a few bands less so.
    """
    L, H, F = w.n_layers, w.n_kv_heads, w.n_bands
    q = np.asarray(qbar, np.float64)
    centre = np.abs(q[..., 0::2] + 1j * q[..., 1::2])
    R = np.stack([rng(w.wid, l, K_QABS).uniform(0.85, 1.0, (H, F)) for l in range(L)])
    return (centre / R).astype(np.float32)


def head_kv_numpy(w: Workload, l: int, s: int, mu: np.ndarray):
    """K and V of one (layer, seq) for every KV head, drawn with NumPy.

    Returns (K, V) shaped [H, t_cap, d]: fp32 arrays for "f32", uint16 bf16
    bits for "bf16". Slots at or beyond the sequence length are zero.
    """
    H, d, Tc = w.n_kv_heads, w.head_dim, w.t_cap
    T = int(w.seq_len[s])
    noise = rng(w.wid, l, s, K_KEYNOISE).standard_normal((H, T, d))
    k = (mu[l][:, None, :].astype(np.float64) + w.key_noise * noise).astype(np.float32)
    v = rng(w.wid, l, s, K_VAL).standard_normal((H, T, d)).astype(np.float32)
    K = np.zeros((H, Tc, d), np.float32)
    V = np.zeros((H, Tc, d), np.float32)
    K[:, :T] = k
    V[:, :T] = v
    if w.dtype == "bf16":
        return bf16_bits(K), bf16_bits(V)
    return K, V


def kv_numpy(w: Workload):
    """The whole cache drawn with NumPy (small workloads only): K, V, mu, q_bar."""
    mu, qb, _ = centres(w)
    shp = (w.n_layers, w.n_seq, w.n_kv_heads, w.t_cap, w.head_dim)
    dt = np.float32 if w.dtype == "f32" else np.uint16
    K = np.zeros(shp, dt)
    V = np.zeros(shp, dt)
    for l in range(w.n_layers):
        for s in range(w.n_seq):
            K[l, s], V[l, s] = head_kv_numpy(w, l, s, mu)
    return K, V, mu, qb


# ----------------------------------------------------------------------------
# bulk device draws: torch (only imported when used)
# ----------------------------------------------------------------------------
def kv_torch(w: Workload, device, mu: Optional[np.ndarray] = None, with_values: bool = True):
    """Draw the whole cache on ``device`` layer by layer with torch generators.

    Returns (K, V) as torch tensors [L,S,H,t_cap,d] of dtype float32/bfloat16
    (V is None when ``with_values`` is False). Slots at or beyond each
    sequence's length are zero.
    """
    import torch

    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    if mu is None:
        mu, _, _ = centres(w)
    L, S, H, Tc, d = w.n_layers, w.n_seq, w.n_kv_heads, w.t_cap, w.head_dim
    K = torch.empty((L, S, H, Tc, d), dtype=tdt, device=device)
    V = torch.empty((L, S, H, Tc, d), dtype=tdt, device=device) if with_values else None
    lens = torch.as_tensor(w.seq_len.astype(np.int64), device=device)
    valid = (torch.arange(Tc, device=device)[None, :] < lens[:, None])  # [S, Tc]
    vmask = valid[:, None, :, None]
    for l in range(L):
        g = torch.Generator(device=device)
        g.manual_seed(torch_seed(w.wid, l, K_KEYNOISE))
        mul = torch.as_tensor(mu[l], device=device)[None, :, None, :]
        x = torch.randn((S, H, Tc, d), generator=g, device=device, dtype=torch.float32)
        x.mul_(w.key_noise).add_(mul)
        x.mul_(vmask)
        K[l].copy_(x.to(tdt))
        if with_values:
            g.manual_seed(torch_seed(w.wid, l, K_VAL))
            x = torch.randn((S, H, Tc, d), generator=g, device=device, dtype=torch.float32)
            x.mul_(vmask)
            V[l].copy_(x.to(tdt))
        del x
    return K, V


def periodic_tokens_torch(w: Workload, event: int, first_pos: np.ndarray, mu0: np.ndarray,
                          drift_dir: np.ndarray, device):
    """New keys/values for the periodic workload: ``new_per_event`` tokens per head.

    Token at absolute position p of (layer l, KV head h) has centre
    mu0[l,h] + drift * (p / 1000) * drift_dir[l,h]; sequence s's new tokens sit
    at positions first_pos[s] .. first_pos[s] + new_per_event - 1.
    Returns (K_new, V_new, pos_new) as [L,S,H,n,d] tensors and int32 [S,n].
    """
    import torch

    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    L, S, H, d, n = w.n_layers, w.n_seq, w.n_kv_heads, w.head_dim, w.new_per_event
    pos = torch.as_tensor(first_pos.astype(np.int64), device=device)[:, None] + \
        torch.arange(n, device=device)[None, :]                       # [S, n]
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(w.wid, event, K_NEWKEY))
    x = torch.randn((L, S, H, n, d), generator=g, device=device, dtype=torch.float32)
    mu_t = torch.as_tensor(mu0, device=device)[:, None, :, None, :]   # [L,1,H,1,d]
    dr_t = torch.as_tensor(drift_dir, device=device)[:, None, :, None, :]
    age = (pos.to(torch.float32) * (w.drift / 1000.0))[None, :, None, :, None]
    x.mul_(w.key_noise).add_(mu_t).add_(age * dr_t)
    g.manual_seed(torch_seed(w.wid, event, K_NEWVAL))
    v = torch.randn((L, S, H, n, d), generator=g, device=device, dtype=torch.float32)
    return x.to(tdt), v.to(tdt), pos.to(torch.int32)


def periodic_prompt_torch(w: Workload, mu0: np.ndarray, drift_dir: np.ndarray, device):
    """Prompt keys/values of the periodic workload, placed at slots 0..P_s-1."""
    import torch

    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    L, S, H, Tc, d = w.n_layers, w.n_seq, w.n_kv_heads, w.t_cap, w.head_dim
    pos = torch.arange(Tc, device=device)
    lens = torch.as_tensor(w.prompt_len.astype(np.int64), device=device)
    valid = (pos[None, :] < lens[:, None])[None, :, None, :, None]   # [1,S,1,Tc,1]
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed(w.wid, 0, K_KEYNOISE))
    x = torch.randn((L, S, H, Tc, d), generator=g, device=device, dtype=torch.float32)
    mu_t = torch.as_tensor(mu0, device=device)[:, None, :, None, :]
    dr_t = torch.as_tensor(drift_dir, device=device)[:, None, :, None, :]
    age = (pos.to(torch.float32) * (w.drift / 1000.0))[None, None, None, :, None]
    x.mul_(w.key_noise).add_(mu_t).add_(age * dr_t).mul_(valid)
    g.manual_seed(torch_seed(w.wid, 0, K_VAL))
    v = torch.randn((L, S, H, Tc, d), generator=g, device=device, dtype=torch.float32).mul_(valid)
    return x.to(tdt), v.to(tdt)


# ----------------------------------------------------------------------------
# generic draws for edge-case and selector tests
# ----------------------------------------------------------------------------
def random_scores(seed: int, shape: Sequence[int], ties: float = 0.0, specials: bool = False) -> np.ndarray:
    """fp32 score arrays for selector tests.

    ``ties`` is the fraction of entries copied from another entry (exact ties);
    ``specials`` plants NaN, +-inf, +0.0 and -0.0 values.
    """
    r = rng(90, seed)
    x = r.standard_normal(shape).astype(np.float32)
    flat = x.reshape(-1)
    n = flat.size
    if ties > 0 and n > 1:
        m = int(ties * n)
        dst = r.integers(0, n, m)
        src = r.integers(0, n, m)
        flat[dst] = flat[src]
    if specials and n >= 8:
        idx = r.choice(n, size=min(n, max(8, n // 50)), replace=False)
        vals = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, np.nan, 0.0, -0.0], np.float32)
        flat[idx] = vals[np.arange(idx.size) % vals.size]
    return x


def random_kept(seed: int, T: int, n: int) -> np.ndarray:
    """A sorted random subset of n slots of [0, T) (int32)."""
    r = rng(91, seed)
    return np.sort(r.choice(T, size=n, replace=False)).astype(np.int32)

"""Throughput of the KV-eviction hot path on one MI355X.

One step = one full eviction pass over the Qwen3-8B-shaped 32K cache
(36 layers x 8 sequences x 8 KV heads, head_dim 128, bf16, T=32768, prompt
1024, budget 3072, recent window 128, RoPE theta 1e6, 17 geometric offsets):
tri_score -> kv_select_topk -> kv_compact, all on device-resident inputs.
The random-eviction pass (kv_select_random -> kv_compact) over the same
cache is timed in the same run and reported beside it.

Prints one JSON line. `value` is KV entries (layer, seq, KV head, slot)
scored+selected+compacted per second. The roofline block is for the
dominant kernel (tri_score): algorithmic bytes per launch (each key row read
once + one fp32 score written per entry) over its mean launch time measured
with HIP events on the launch stream. `cpu_baseline` times the fp64 NumPy
oracle on the same pass on the host, one worker process per available CPU;
`cpu_protocol` times it on every workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, vendor figure
METRIC = "KV tokens scored+selected+compacted/sec and HBM GB/s (% peak), Qwen3-8B 32K"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=36, help="layers of the full-pass workload (36 = full size)")
    ap.add_argument("--no-cpu", action="store_true", help="skip timing the CPU oracle")
    ap.add_argument("--no-random", action="store_true", help="skip the random-eviction pass")
    ap.add_argument("--no-generation", action="store_true",
                    help="skip the simulated 256-event generation of the periodic workload")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the 512-slot, one-layer and ragged-batch workloads")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="run one elementwise copy of known size then exit after one pass (for HBM counter runs)")
    ap.add_argument("--pmc-probe-next", action="store_true",
                    help="like --pmc-probe, then one launch of each next-row kernel over the same cache; prints "
                         "their algorithmic bytes as one JSON line")
    return ap.parse_args()


def pmc_probe_next(w, K, qb, qbd, seq, plen, tcur, scores, kept, nk, b_cap, dev):
    """One launch of each next-row kernel over the full-pass cache, in this order, for the HBM
    counter runs; returns [kernel-name fragment, algorithmic read bytes, algorithmic write bytes]
    per dispatch."""
    import numpy as np
    import torch

    import eviction_long_reasoning_amd as kv
    from workloads import query_head_centres, query_magnitudes, workload
    L, S, H, T, d = K.shape
    e = K.element_size()
    n = L * S * H * T
    heads = L * S * H
    out = []
    kv.tri_score(K, qbd, tcur, seq, w.theta, w.deltas, out=scores,
                 qabs=torch.from_numpy(query_magnitudes(w, qb)).to(dev))
    out.append(["score_stream_kernel<true, 16, true, true>", n * d * e, n * 4])
    kv.tri_score_rotated(K, qbd, tcur, seq, w.theta, w.deltas, out=scores)
    out.append(["score_rotated_kernel<true, 16, false, 0, false>", n * d * e, n * 4])
    bs, bps = 16, T // 16
    g = torch.Generator(device="cpu")
    g.manual_seed(7)
    table = torch.randperm(S * bps, generator=g).view(S, bps).to(torch.int32).to(dev)
    kv.tri_score_rotated(K.view(L, S * bps, H, bs, d), qbd, tcur, seq, w.theta, w.deltas, block_table=table,
                         out=scores, head_major=True)
    out.append(["score_rotated_kernel<true, 16, false, 2, false>", n * d * e + L * H * S * bps * 4, n * 4])
    G = w.group
    nu = torch.from_numpy(query_head_centres(workload(w.wid, L=L, q_mode="group-mean"))).to(dev)
    zmax, head = kv.tri_score_gqa(K, nu, tcur, seq, w.theta, w.deltas)
    out.append(["gqa_stream_kernel<true, 16, true, false, 4>", n * d * e, n * 4 * G])
    out.append(["gqa_finish_kernel<4>", n * 4 * G, n * 4])
    kv.kv_select_union(head, zmax, seq, plen, w.budget, w.recent, w.prompt_cap(), b_cap=b_cap, kept=kept, n_kept=nk)
    out.append(["select_kernel<1024, 32, 2>", n * 4 * (G + 1), heads * b_cap * 4])
    del zmax, head
    kv.kv_select_random((L, S, H, T), seq, plen, w.budget, w.recent, w.prompt_cap(), 1, 0, b_cap=b_cap, kept=kept,
                        n_kept=nk)
    out.append(["select_stream_kernel<1, 512>", 0, heads * b_cap * 4])
    Sl, Tl = S // 4, 4 * T
    kl = torch.empty((L, Sl, H, b_cap), dtype=torch.int32, device=dev)
    nkl = torch.empty((Sl,), dtype=torch.int32, device=dev)
    kv.kv_select_topk(scores.view(L, Sl, H, Tl), i32_dev(np.full(Sl, Tl), dev), i32_dev(np.full(Sl, w.prompt_len[0]), dev),
                      w.budget, w.recent, w.prompt_cap(), b_cap=b_cap, kept=kl, n_kept=nkl)
    out.append(["select_stream_kernel<0, 1024>", n * 4, L * Sl * H * b_cap * 4])
    zmax, head = kv.tri_score_gqa_rotated(K.view(L, S * bps, bs, H, d), nu, tcur, seq, w.theta, w.deltas,
                                          block_table=table)
    out.append(["gqa_rotated_kernel<true, 16, false, 1, false, 4>", n * d * e + L * H * S * bps * 4, n * 4 * G])
    out.append(["gqa_finish_kernel<4>", n * 4 * G, n * 4])
    del zmax, head
    torch.cuda.synchronize(dev)
    return {"next_row_dispatches": out}


def i32_dev(a, dev):
    import numpy as np
    import torch
    return torch.as_tensor(np.asarray(a, np.int32), device=dev)


def algorithmic_bytes(w, n_kept_per_head: int):
    """Per-pass algorithmic bytes of each kernel (one read of every key row, one score
    write and read, kept rows of K and V read and written, index and position traffic)."""
    e, d = w.elem_bytes, w.head_dim
    n_entries = w.entries
    n_heads = w.n_heads_total
    n_kept = n_heads * n_kept_per_head
    score = n_entries * (d * e + 4)
    select = n_entries * 4 + n_heads * w.b_cap() * 4
    compact = n_kept * (4 * d * e + 4 + 4) + n_heads * 0
    rnd_select = n_heads * w.b_cap() * 4
    return dict(score=score, select=select, compact=compact, random_select=rnd_select)


def counter_traffic():
    """HBM bytes per tri_score launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary
    (already scaled by the copy calibration), or None when the score kernel's sources have changed
    since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "tri_score_full_pass_hbm_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = hashlib.sha256()
    for f in ("score.hip", "score_params.hpp"):
        h.update(open(os.path.join(ROOT, "eviction_long_reasoning_amd", "csrc", f), "rb").read())
    m = re.search(r"sha256 `([0-9a-f]+)`", text)
    row = re.search(r"^\| `void score_stream_kernel<[^`]*>` \| ([0-9.]+) \| ([0-9.]+) \|", text, re.M)
    if not m or m.group(1) != h.hexdigest() or not row:
        return None
    return (float(row.group(1)) + float(row.group(2))) * 1e9


def percentiles(ms):
    import numpy as np
    q = np.percentile(np.asarray(ms, np.float64), [10, 50, 90])
    return {"p10_ms": float(q[0]), "median_ms": float(q[1]), "p90_ms": float(q[2]), "reps": len(ms)}


def kept_jaccard(ka, kb, t_cap):
    """Mean over heads of |A & B| / |A | B| for two [..., b_cap] kept lists (-1 padded)."""
    import torch
    bc = ka.shape[-1]

    def mask(k):
        idx = k.reshape(-1, bc).long()
        idx = torch.where(idx < 0, torch.full_like(idx, t_cap), idx)
        m = torch.zeros((idx.shape[0], t_cap + 1), dtype=torch.bool, device=k.device)
        m.scatter_(1, idx, True)
        return m[:, :t_cap]
    a, b = mask(ka), mask(kb)
    inter = (a & b).sum(1).double()
    union = (a | b).sum(1).double().clamp(min=1)
    return float((inter / union).mean())


def other_workloads(args, dev):
    """Whole passes over the pages' other single-GPU shapes, each rep timed alone with HIP events:
    one 512-slot fp32 head (launch latency), one 8-head layer of 32768 slots with the 256 MB
    last-level cache flushed before every rep (cold) or not (warm), and 128 ragged sequences
    scored and randomly evicted (the two passes' ratio and kept-set overlap)."""
    import numpy as np
    import torch

    import eviction_long_reasoning_amd as kv
    from workloads import centres, kv_torch, workload
    reps = max(20, args.steps)
    i32 = lambda a: torch.as_tensor(np.asarray(a, np.int32), device=dev)
    flush_buf = torch.empty((1 << 28,), dtype=torch.float32, device=dev)   # 1 GiB

    def timed(fn, cold=False, host=False):
        """Per-rep milliseconds between two events around fn(). The GPU is kept busy before the
        first event (the cache flush, or a bounded spin) so that the host has queued the whole pass
        when it starts: the events then time the device alone. host=True starts each rep on an idle
        GPU, so the time includes the host's launch path."""
        for _ in range(args.warmup):
            fn()
        out = []
        for i in range(reps):
            if cold:
                flush_buf.fill_(float(i))
            elif not host:
                torch.cuda._sleep(100000)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record()
            fn()
            e[1].record()
            torch.cuda.synchronize(dev)
            out.append(e[0].elapsed_time(e[1]))
        return out

    def prepare(wid):
        w = workload(wid)
        mu, qb, _ = centres(w)
        K, V = kv_torch(w, dev, mu)
        L, S, H = w.n_layers, w.n_seq, w.n_kv_heads
        c = dict(w=w, K=K, V=V, qb=torch.from_numpy(qb).to(dev), seq=i32(w.seq_len), plen=i32(w.prompt_len),
                 tcur=i32(w.t_cur), scores=torch.empty((L, S, H, w.t_cap), dtype=torch.float32, device=dev),
                 kept=torch.empty((L, S, H, w.b_cap()), dtype=torch.int32, device=dev),
                 nk=torch.empty((S,), dtype=torch.int32, device=dev),
                 Ko=torch.empty((L, S, H, w.out_cap, w.head_dim), dtype=K.dtype, device=dev),
                 Po=torch.empty((L, S, H, w.out_cap), dtype=torch.int32, device=dev))
        c["Vo"] = torch.empty_like(c["Ko"])
        c["ws"] = torch.empty((kv.select_workspace_bytes(L, S, H, w.t_cap, w.b_cap()),), dtype=torch.uint8, device=dev)
        return c

    def scored(c):
        w = c["w"]
        kv.tri_score(c["K"], c["qb"], c["tcur"], c["seq"], w.theta, w.deltas, out=c["scores"])
        kv.kv_select_topk(c["scores"], c["seq"], c["plen"], w.budget, w.recent, w.prompt_cap(), b_cap=w.b_cap(),
                          kept=c["kept"], n_kept=c["nk"], workspace=c["ws"])
        kv.kv_compact(c["K"], c["V"], c["kept"], c["nk"], c["seq"], w.out_cap, K_out=c["Ko"], V_out=c["Vo"],
                      pos_out=c["Po"])

    def random(c):
        w = c["w"]
        kv.kv_select_random(tuple(c["scores"].shape), c["seq"], c["plen"], w.budget, w.recent, w.prompt_cap(),
                            w.seed_random, 0, b_cap=w.b_cap(), kept=c["kept"], n_kept=c["nk"], workspace=c["ws"])
        kv.kv_compact(c["K"], c["V"], c["kept"], c["nk"], c["seq"], w.out_cap, K_out=c["Ko"], V_out=c["Vo"],
                      pos_out=c["Po"])

    def pass_bytes(c, with_score):
        w = c["w"]
        e, d = c["K"].element_size(), w.head_dim
        rows = int(c["nk"].sum()) * w.n_layers * w.n_kv_heads
        b = rows * (4 * d * e + 8) + w.n_heads_total * w.b_cap() * 4
        return b + (w.entries * (d * e + 8) if with_score else 0)

    res = {}
    c = prepare(1)
    t, tc, th = timed(lambda: scored(c)), timed(lambda: scored(c), cold=True), timed(lambda: scored(c), host=True)
    res["fp32_512_slots"] = {"workload": c["w"].name, "entries": c["w"].entries, "scored_pass": percentiles(t),
                             "scored_pass_cold": percentiles(tc), "scored_pass_host_inclusive": percentiles(th)}
    print(f"[bench] 512-slot fp32 head: scored pass {np.median(t) * 1e3:.1f} us on the device "
          f"({np.median(tc) * 1e3:.1f} us cold), {np.median(th) * 1e3:.1f} us from an idle GPU (host launch path "
          f"included)", file=sys.stderr, flush=True)
    del c
    c = prepare(2)
    warm, cold = timed(lambda: scored(c)), timed(lambda: scored(c), cold=True)
    b2 = pass_bytes(c, True)
    res["one_layer_32k"] = {"workload": c["w"].name, "entries": c["w"].entries, "algorithmic_bytes": b2,
                            "warm": percentiles(warm), "cold": percentiles(cold),
                            "cold_gbs": b2 / (np.median(cold) * 1e-3) / 1e9}
    print(f"[bench] one 8-head layer of 32768 slots: warm {np.median(warm):.4f} ms, cold {np.median(cold):.4f} ms",
          file=sys.stderr, flush=True)
    del c
    c = prepare(5)
    ts = timed(lambda: scored(c))
    bs_ = pass_bytes(c, True)
    ks = c["kept"].clone()
    tr = timed(lambda: random(c))
    br = pass_bytes(c, False)
    jac = kept_jaccard(ks, c["kept"], c["w"].t_cap)
    ms_s, ms_r = float(np.median(ts)), float(np.median(tr))
    res["ragged_128_seqs"] = {"workload": c["w"].name, "entries": c["w"].entries,
                              "scored_pass": percentiles(ts), "scored_gbs": bs_ / (ms_s * 1e-3) / 1e9,
                              "scored_entries_per_s": c["w"].entries / (ms_s * 1e-3),
                              "random_pass": percentiles(tr), "random_gbs": br / (ms_r * 1e-3) / 1e9,
                              "random_over_scored_time": ms_r / ms_s, "mean_kept_jaccard": jac}
    print(f"[bench] 128 ragged sequences: scored {ms_s:.3f} ms, random {ms_r:.3f} ms, mean Jaccard {jac:.3f}",
          file=sys.stderr, flush=True)
    del c, ks, flush_buf
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------------------------------------
# The CPU oracle, timed on the host's cores: one worker process per available CPU, each working
# through (layer, seq, KV head) units -- score (the literal RoPE dot product or the folded form),
# lexsort top-n select, gather of the kept K/V rows -- on the same bf16 bits the GPU reads, handed
# over through shared memory. The pool is started before the GPU is touched.
# ------------------------------------------------------------------------------------------------
def _oracle_unit(task):
    """One (layer, seq, KV head) unit of the oracle (runs in a worker process); returns T."""
    import numpy as np
    from multiprocessing import shared_memory
    from threadpoolctl import threadpool_limits

    import oracle
    from workloads import bf16_to_f32

    shm_name, kv_shape, kv_dtype, pos_off, unit, T, P, B, R, qbar, t, theta, deltas, form = task
    shm = shared_memory.SharedMemory(name=shm_name)
    try:
        n_units, t_cap, d = kv_shape
        dt = np.uint16 if kv_dtype == "bf16" else np.float32
        KV = np.ndarray((2, n_units, t_cap, d), dtype=dt, buffer=shm.buf)
        pos = None
        if pos_off >= 0:
            pos = np.ndarray((n_units, t_cap), dtype=np.int32, buffer=shm.buf, offset=pos_off)[unit, :T]
        with threadpool_limits(1):
            k, v = KV[0, unit, :T], KV[1, unit, :T]
            if kv_dtype == "bf16":
                k, v = bf16_to_f32(k), bf16_to_f32(v)
            k = k.astype(np.float64)
            score = oracle.score_literal if form == "literal" else oracle.score_folded
            sc = score(k, pos, qbar, t, theta, deltas)
            kept = oracle.select_topk(sc, T, P, B, R)
            oracle.compact(k, v, pos, kept)
        del KV, k, v
    finally:
        shm.close()
    return int(T)


class OracleTimer:
    """The worker pool and the per-workload timing of the oracle."""

    def __init__(self):
        import multiprocessing as mp
        self.cores = len(os.sched_getaffinity(0))
        self.pool = mp.get_context("spawn").Pool(self.cores)
        self.pool.map(int, range(self.cores))   # workers up and importing before the GPU is used

    def close(self):
        self.pool.close()
        self.pool.join()

    def run(self, K, V, pos, units, form):
        """Time the oracle over ``units`` = [(index into K/V, T, P, B, R, qbar, t, theta, deltas)];
        K, V are host arrays [n, t_cap, d] (bf16 bits or fp32), pos None or int32 [n, t_cap].
        Returns (seconds, entries)."""
        import numpy as np
        from multiprocessing import shared_memory
        n, t_cap, d = K.shape
        kv_bytes = 2 * K.nbytes
        size = kv_bytes + (n * t_cap * 4 if pos is not None else 0)
        shm = shared_memory.SharedMemory(create=True, size=size)
        try:
            buf = np.ndarray((2, n, t_cap, d), dtype=K.dtype, buffer=shm.buf)
            buf[0], buf[1] = K, V
            pos_off = -1
            if pos is not None:
                pos_off = kv_bytes
                np.ndarray((n, t_cap), dtype=np.int32, buffer=shm.buf, offset=pos_off)[...] = pos
            kd = "bf16" if K.dtype == np.uint16 else "f32"
            tasks = [(shm.name, (n, t_cap, d), kd, pos_off, u[0], *u[1:], form) for u in units]
            del buf
            t0 = time.perf_counter()
            done = self.pool.map(_oracle_unit, tasks, chunksize=1)
            dt = time.perf_counter() - t0
        finally:
            shm.close()
            shm.unlink()
        return dt, int(sum(done))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        return None


def host_bits(t):
    """A device tensor's bytes on the host as uint16 (bf16) or fp32 NumPy."""
    import numpy as np
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def oracle_protocol(timer, dev, args, w3, K3, V3, qb3):
    """The oracle on every workload: literal score on workloads 1, 2 and 5 and on one layer of
    workload 3 (extrapolated to its 36 layers); folded score on all five -- workload 3 whole (a
    layer at a time), workload 4 on one steady-state event (extrapolated to its 256 events)."""
    import numpy as np
    import torch

    from workloads import centres, kv_numpy, kv_torch, workload
    res = {}

    def units_of(w, qb, layers, t=None):
        out = []
        for li, l in enumerate(layers):
            for s in range(w.n_seq):
                for h in range(w.n_kv_heads):
                    tt = int(w.t_cur[s]) if t is None else int(t[s])
                    out.append(((li * w.n_seq + s) * w.n_kv_heads + h, int(w.seq_len[s]), int(w.prompt_len[s]),
                                w.budget, w.recent, qb[l, h].astype(np.float64), tt, w.theta, w.deltas))
        return out

    def record(name, w, forms, run_one, scale=1.0, note=""):
        entry = {"workload": w.name}
        for form in forms:
            sec, n = run_one(form)
            entry[form] = {"seconds": sec * scale, "entries": int(n * scale), "entries_per_s": n / sec,
                           "measured_seconds": sec, "measured_entries": n}
        if note:
            entry["note"] = note
        res[name] = entry
        print(f"[bench] oracle {name}: " + ", ".join(f"{f} {entry[f]['entries_per_s']:.3g} entries/s"
                                                     for f in forms), file=sys.stderr, flush=True)

    # workload 1: the whole head from NumPy
    w1 = workload(1)
    K1, V1, _, qb1 = kv_numpy(w1)
    record("tiny_fp32_512", w1, ("literal", "folded"),
           lambda f: timer.run(K1.reshape(-1, w1.t_cap, w1.head_dim), V1.reshape(-1, w1.t_cap, w1.head_dim), None,
                               units_of(w1, qb1, [0]), f))
    # workload 2: one 8-head layer drawn on the device
    w2 = workload(2)
    mu2, qb2, _ = centres(w2)
    K2, V2 = kv_torch(w2, dev, mu2)
    k2, v2 = host_bits(K2).reshape(-1, w2.t_cap, w2.head_dim), host_bits(V2).reshape(-1, w2.t_cap, w2.head_dim)
    del K2, V2
    record("one_layer_32k", w2, ("literal", "folded"), lambda f: timer.run(k2, v2, None, units_of(w2, qb2, [0]), f))
    del k2, v2
    # workload 5: 128 ragged sequences
    w5 = workload(5)
    mu5, qb5, _ = centres(w5)
    K5, V5 = kv_torch(w5, dev, mu5)
    k5, v5 = host_bits(K5).reshape(-1, w5.t_cap, w5.head_dim), host_bits(V5).reshape(-1, w5.t_cap, w5.head_dim)
    del K5, V5
    torch.cuda.empty_cache()
    record("ragged_128_seqs", w5, ("literal", "folded"), lambda f: timer.run(k5, v5, None, units_of(w5, qb5, [0]), f))
    del k5, v5
    # workload 3: folded over all layers, streamed a layer at a time; literal on layer 0 (x36)
    L3 = K3.shape[0]

    def w3_folded(form):
        sec = n = 0
        for l in range(L3):
            k, v = host_bits(K3[l]).reshape(-1, w3.t_cap, w3.head_dim), host_bits(V3[l]).reshape(-1, w3.t_cap,
                                                                                                 w3.head_dim)
            dt, dn = timer.run(k, v, None, units_of(w3, qb3, [l]), form)
            sec, n = sec + dt, n + dn
        return sec, n
    record("full_pass_32k", w3, ("folded",), w3_folded)
    k, v = host_bits(K3[0]).reshape(-1, w3.t_cap, w3.head_dim), host_bits(V3[0]).reshape(-1, w3.t_cap, w3.head_dim)
    record("full_pass_32k_literal_layer0", w3, ("literal",), lambda f: timer.run(k, v, None, units_of(w3, qb3, [0]), f),
           scale=L3, note=f"layer 0 measured, seconds and entries scaled x{L3} to the whole pass")
    del k, v
    # workload 4: one steady-state event (every head at B + 128 entries, gappy positions)
    w4 = workload(4)
    w4f = workload(4, seq_len=np.full(w4.n_seq, w4.t_cap, np.int32))
    mu4, qb4, _ = centres(w4f)
    K4, V4 = kv_torch(w4f, dev, mu4)
    k4, v4 = host_bits(K4).reshape(-1, w4f.t_cap, w4f.head_dim), host_bits(V4).reshape(-1, w4f.t_cap, w4f.head_dim)
    del K4, V4
    torch.cuda.empty_cache()
    gap = np.random.default_rng(4).integers(1, 3, (k4.shape[0], w4f.t_cap)).astype(np.int64)
    pos4 = np.cumsum(gap, axis=1).astype(np.int32)          # ascending, gappy (events evict slots)
    t4 = np.full(w4f.n_seq, int(pos4.max()) + 1)
    record("periodic_event", w4f, ("folded",),
           lambda f: timer.run(k4, v4, pos4, units_of(w4f, qb4, range(w4f.n_layers), t4), f), scale=w4.n_events,
           note=f"one steady-state event measured (every head at {w4f.t_cap} entries, gappy positions); seconds and "
                f"entries scaled x{w4.n_events} to the simulated generation's events")
    del k4, v4
    return res


def periodic_workload(args, dev, time_launches, mu4, qb4):
    """The gpt-oss-20b-shaped periodic eviction: one steady-state event (every head at B + 128 = 2176
    entries) kernel by kernel and as whole passes -- scored (tri_score with positions, top-B) or
    random, each with the gather into a second buffer or in-place hole filling -- then a whole
    simulated 32768-token generation: 256 events, 128 tokens appended to every sequence between
    them (untimed), each event's pass timed alone on the device."""
    import numpy as np
    import torch

    import eviction_long_reasoning_amd as kv
    from workloads import centres, kv_torch, periodic_prompt_torch, periodic_tokens_torch, workload
    i32 = lambda a: torch.as_tensor(np.asarray(a, np.int32), device=dev)
    w4 = workload(4)
    w4f = workload(4, seq_len=np.full(w4.n_seq, w4.t_cap, np.int32))
    L, S, H, Tc, d = w4f.n_layers, w4f.n_seq, w4f.n_kv_heads, w4f.t_cap, w4f.head_dim
    K4, V4 = kv_torch(w4f, dev, mu4)
    pos4 = torch.arange(Tc, dtype=torch.int32, device=dev).expand(L, S, H, Tc).contiguous()
    e = K4.element_size()
    row = d * e
    seq4, plen4 = i32(w4f.seq_len), i32(w4f.prompt_len)
    qb4d, tcur4 = torch.from_numpy(qb4).to(dev), i32(np.full(S, Tc))   # the next position
    b_cap, out4 = w4f.b_cap(), w4f.budget
    heads = L * S * H
    sc4 = torch.empty((L, S, H, Tc), dtype=torch.float32, device=dev)
    kept4 = torch.empty((L, S, H, b_cap), dtype=torch.int32, device=dev)
    nk4 = torch.empty((S,), dtype=torch.int32, device=dev)
    ws_s = torch.empty((kv.score_workspace_bytes(L, S, H, Tc, d, K4.dtype, len(w4f.deltas)),), dtype=torch.uint8,
                       device=dev)
    ws_k = torch.empty((kv.select_workspace_bytes(L, S, H, Tc, b_cap),), dtype=torch.uint8, device=dev)
    Ko4 = torch.empty((L, S, H, out4, d), dtype=K4.dtype, device=dev)
    Vo4 = torch.empty_like(Ko4)
    Po4 = torch.empty((L, S, H, out4), dtype=torch.int32, device=dev)

    def score(K, pos, seq, tcur, out, ws):
        kv.tri_score(K, qb4d, tcur, seq, w4f.theta, w4f.deltas, pos=pos, out=out, workspace=ws)

    def draw(seq, plen, pos, ev, kept, nk, ws):
        kv.kv_select_random(tuple(pos.shape), seq, plen, w4f.budget, w4f.recent, w4f.prompt_cap(), w4f.seed_random,
                            ev, pos=pos, b_cap=b_cap, kept=kept, n_kept=nk, workspace=ws)

    # kernel by kernel
    score4_ms = time_launches(lambda: score(K4, pos4, seq4, tcur4, sc4, ws_s))
    topk4_ms = time_launches(lambda: kv.kv_select_topk(sc4, seq4, plen4, w4f.budget, w4f.recent, w4f.prompt_cap(),
                                                       b_cap=b_cap, kept=kept4, n_kept=nk4, workspace=ws_k))
    sel4_ms = time_launches(lambda: draw(seq4, plen4, pos4, 1, kept4, nk4, ws_k))
    gather_ms = time_launches(lambda: kv.kv_compact(K4, V4, kept4, nk4, seq4, out4, pos=pos4, K_out=Ko4, V_out=Vo4,
                                                    pos_out=Po4))
    n = w4f.entries
    n_kept = int(nk4.sum()) * L * H
    nkh = nk4.to(torch.int64)[None, :, None, None]
    movers = int(((kept4.to(torch.int64) >= nkh) & (torch.arange(b_cap, device=dev) < nkh)).sum())
    bytes_score = n * (row + 4 + 4)                       # key row and position read, score written
    bytes_topk = n * 4 + heads * b_cap * 4                 # scores read, kept list written
    bytes_draw = n * 4 + heads * b_cap * 4                 # positions read, kept list written
    bytes_gather = n_kept * (4 * row + 4 + 4 + 4)          # K, V rows read and written; index, position
    bytes_inplace = movers * (4 * row + 4 + 4)             # moved rows only

    # whole passes over the steady-state event; the in-place passes start each rep from a copy of
    # the event's cache (the copy is outside the timed region)
    Ks, Vs, Ps = K4.clone(), V4.clone(), pos4.clone()

    def restore():
        K4.copy_(Ks)
        V4.copy_(Vs)
        pos4.copy_(Ps)

    def scored(inplace):
        score(K4, pos4, seq4, tcur4, sc4, ws_s)
        kv.kv_select_topk(sc4, seq4, plen4, w4f.budget, w4f.recent, w4f.prompt_cap(), b_cap=b_cap, kept=kept4,
                          n_kept=nk4, workspace=ws_k)
        compact(inplace)

    def rnd(inplace):
        draw(seq4, plen4, pos4, 1, kept4, nk4, ws_k)
        compact(inplace)

    def compact(inplace):
        if inplace:
            kv.kv_compact_inplace(K4, V4, kept4, nk4, seq4, pos=pos4)
        else:
            kv.kv_compact(K4, V4, kept4, nk4, seq4, out4, pos=pos4, K_out=Ko4, V_out=Vo4, pos_out=Po4)

    def pass_ms(fn):
        for _ in range(args.warmup):
            restore()
            fn()
        ms = []
        for _ in range(max(10, args.steps)):
            restore()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize(dev)
            ms.append(ev[0].elapsed_time(ev[1]))
        return percentiles(ms)

    passes = {}
    for name, fn, byts in (("scored_gather", lambda: scored(False), bytes_score + bytes_topk + bytes_gather),
                           ("scored_in_place", lambda: scored(True), bytes_score + bytes_topk + bytes_inplace),
                           ("random_gather", lambda: rnd(False), bytes_draw + bytes_gather),
                           ("random_in_place", lambda: rnd(True), bytes_draw + bytes_inplace)):
        st = pass_ms(fn)
        passes[name] = {"ms": st, "algorithmic_bytes": byts, "gbs": byts / (st["median_ms"] * 1e-3) / 1e9,
                        "entries_per_s": n / (st["median_ms"] * 1e-3)}
    restore()
    del Ks, Vs, Ps, K4, V4, pos4, sc4, Ko4, Vo4, Po4
    torch.cuda.empty_cache()
    print(f"[bench] periodic event, kernels: score (positions) {score4_ms:.3f} ms, top-k {topk4_ms:.3f} ms, random "
          f"select {sel4_ms:.3f} ms, gather {gather_ms:.3f} ms; whole passes (median ms): "
          + ", ".join(f"{k} {v['ms']['median_ms']:.3f}" for k, v in passes.items()), file=sys.stderr, flush=True)

    # the simulated generation: every sequence starts at its prompt; events fire every 128 generated
    # tokens; a sequence whose cache exceeds B is evicted back to B (its other slots copied as they are)
    if args.no_generation:
        return {"workload": w4f.name, "entries_per_event": n,
                "kernels": {"tri_score_with_positions": {"ms": score4_ms, "algorithmic_bytes": bytes_score},
                            "kv_select_topk_ms": topk4_ms, "kv_select_random_ms": sel4_ms,
                            "kv_compact": {"ms": gather_ms, "algorithmic_bytes": bytes_gather}},
                "event_passes": passes, "generation": None}
    P = w4.prompt_len.astype(np.int64)
    mu0, _, dr = centres(w4)
    K0, V0 = periodic_prompt_torch(w4, mu0, dr, dev)
    sc_g = torch.empty((L, S, H, Tc), dtype=torch.float32, device=dev)
    gen = {}
    for mode in ("scored", "random"):
        for inplace in (False, True):
            bufs = [(K0.clone(), V0.clone(), torch.arange(Tc, dtype=torch.int32, device=dev).expand(L, S, H, Tc).contiguous())]
            if not inplace:
                bufs.append((torch.empty_like(K0), torch.empty_like(V0), torch.empty((L, S, H, Tc), dtype=torch.int32,
                                                                                     device=dev)))
            cur, T = 0, P.copy()
            marks, byts, ents = [], 0, 0
            for ev in range(1, w4.n_events + 1):
                Kc, Vc, Pc = bufs[cur]
                Kn, Vn, pn = periodic_tokens_torch(w4, ev, (P + w4.new_per_event * (ev - 1)).astype(np.int32), mu0, dr,
                                                   dev)
                for t0 in np.unique(T):          # sequences at the same length append with one slice
                    idx = torch.as_tensor(np.nonzero(T == t0)[0], device=dev)
                    sl = slice(int(t0), int(t0) + w4.new_per_event)
                    Kc[:, idx, :, sl] = Kn[:, idx]
                    Vc[:, idx, :, sl] = Vn[:, idx]
                    Pc[:, idx, :, sl] = pn[idx][None, :, None, :].expand(L, -1, H, -1)
                T = T + w4.new_per_event
                seq, tcur = i32(T), i32(P + w4.new_per_event * ev)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                if mode == "scored":
                    score(Kc, Pc, seq, tcur, sc_g, ws_s)
                    kv.kv_select_topk(sc_g, seq, i32(P), w4.budget, w4.recent, w4.prompt_cap(), b_cap=b_cap,
                                      kept=kept4, n_kept=nk4, workspace=ws_k)
                else:
                    draw(seq, i32(P), Pc, ev, kept4, nk4, ws_k)
                if inplace:
                    kv.kv_compact_inplace(Kc, Vc, kept4, nk4, seq, pos=Pc)
                else:
                    Ko, Vo, Po = bufs[1 - cur]
                    kv.kv_compact(Kc, Vc, kept4, nk4, seq, Tc, pos=Pc, K_out=Ko, V_out=Vo, pos_out=Po)
                    cur = 1 - cur
                e1.record()
                marks.append((e0, e1))
                nk_h = np.where(T > w4.budget, np.maximum(w4.budget, P), T)   # the partition's n_kept
                n_ev = int(T.sum()) * L * H
                kept_rows = int(nk_h.sum()) * L * H
                ents += n_ev
                if mode == "scored":
                    byts += n_ev * (row + 4 + 4) + n_ev * 4 + heads * b_cap * 4
                else:
                    byts += n_ev * 4 + heads * b_cap * 4
                byts += kept_rows * (4 * row + 12) if not inplace else 0
                T = nk_h.astype(np.int64)
            torch.cuda.synchronize(dev)
            ms = [a.elapsed_time(b) for a, b in marks]
            key = f"{mode}_{'in_place' if inplace else 'gather'}"
            gen[key] = {"events": len(ms), "total_ms": float(np.sum(ms)), "event_ms": percentiles(ms),
                        "entries": ents, "entries_per_s": ents / (np.sum(ms) * 1e-3)}
            if not inplace:
                gen[key]["algorithmic_bytes"] = byts
                gen[key]["gbs"] = byts / (np.sum(ms) * 1e-3) / 1e9
            print(f"[bench] simulated generation, {key}: {len(ms)} events, {np.sum(ms):.1f} ms in total "
                  f"(median event {np.median(ms):.3f} ms)", file=sys.stderr, flush=True)
            del bufs
            torch.cuda.empty_cache()
    return {"workload": w4f.name, "entries_per_event": n,
            "kernels": {"tri_score_with_positions": {"ms": score4_ms, "algorithmic_bytes": bytes_score,
                                                     "gbs": bytes_score / (score4_ms * 1e-3) / 1e9},
                        "kv_select_topk_ms": topk4_ms, "kv_select_random_ms": sel4_ms,
                        "kv_compact": {"ms": gather_ms, "algorithmic_bytes": bytes_gather,
                                       "gbs": bytes_gather / (gather_ms * 1e-3) / 1e9},
                        "in_place_rows_moved": movers, "in_place_algorithmic_bytes": bytes_inplace},
            "event_passes": passes, "generation": gen}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the KV-eviction path runs on one GPU; --gpus must be 1 "
                                   "(the path shards per (layer, seq, KV head) with no exchange)"}))
        sys.exit(2)
    # the oracle's worker processes start before anything touches the GPU
    timer = None if (args.no_cpu or args.pmc_probe or args.pmc_probe_next) else OracleTimer()

    import numpy as np
    import torch

    import eviction_long_reasoning_amd as kv
    from workloads import centres, kv_torch, workload

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workload(3, L=args.layers)
    L, S, H, Tc, d = w.n_layers, w.n_seq, w.n_kv_heads, w.t_cap, w.head_dim
    print(f"[bench] generating {w.name}: L={L} S={S} H={H} T={Tc} d={d} bf16", file=sys.stderr, flush=True)
    mu, qb, _ = centres(w)
    K, V = kv_torch(w, dev, mu)
    i32 = lambda a: torch.as_tensor(np.asarray(a, np.int32), device=dev)
    seq, plen, tcur = i32(w.seq_len), i32(w.prompt_len), i32(w.t_cur)
    qbd = torch.from_numpy(qb).to(dev)
    b_cap, out_cap = w.b_cap(), w.out_cap
    scores = torch.empty((L, S, H, Tc), dtype=torch.float32, device=dev)
    kept = torch.empty((L, S, H, b_cap), dtype=torch.int32, device=dev)
    nk = torch.empty((S,), dtype=torch.int32, device=dev)
    Ko = torch.empty((L, S, H, out_cap, d), dtype=K.dtype, device=dev)
    Vo = torch.empty_like(Ko)
    Po = torch.empty((L, S, H, out_cap), dtype=torch.int32, device=dev)
    ws_score = torch.empty((kv.score_workspace_bytes(L, S, H, Tc, d, K.dtype, len(w.deltas)),), dtype=torch.uint8,
                           device=dev)
    ws_sel = torch.empty((kv.select_workspace_bytes(L, S, H, Tc, b_cap),), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize(dev)
    print("[bench] inputs resident", file=sys.stderr, flush=True)

    if args.pmc_probe or args.pmc_probe_next:
        # elementwise copy of known size (reads 4 GiB, writes 4 GiB) to scale HBM counters
        x = torch.ones(1 << 30, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        torch.mul(x, 1.0, out=y)
        del x, y
        kv.tri_score(K, qbd, tcur, seq, w.theta, w.deltas, out=scores)
        kv.kv_select_topk(scores, seq, plen, w.budget, w.recent, w.prompt_cap(), b_cap=b_cap, kept=kept, n_kept=nk)
        kv.kv_compact(K, V, kept, nk, seq, out_cap, K_out=Ko, V_out=Vo, pos_out=Po)
        torch.cuda.synchronize(dev)
        if args.pmc_probe_next:
            print(json.dumps(pmc_probe_next(w, K, qb, qbd, seq, plen, tcur, scores, kept, nk, b_cap, dev)), flush=True)
        print("[bench] pmc probe done", file=sys.stderr, flush=True)
        return

    def scored_pass(ev=None):
        if ev: ev[0].record()
        kv.tri_score(K, qbd, tcur, seq, w.theta, w.deltas, out=scores, workspace=ws_score)
        if ev: ev[1].record()
        kv.kv_select_topk(scores, seq, plen, w.budget, w.recent, w.prompt_cap(), b_cap=b_cap, kept=kept, n_kept=nk,
                          workspace=ws_sel)
        if ev: ev[2].record()
        kv.kv_compact(K, V, kept, nk, seq, out_cap, K_out=Ko, V_out=Vo, pos_out=Po)
        if ev: ev[3].record()

    def random_pass(event, ev=None):
        if ev: ev[0].record()
        kv.kv_select_random((L, S, H, Tc), seq, plen, w.budget, w.recent, w.prompt_cap(), 0x5EED000000000003,
                            event, b_cap=b_cap, kept=kept, n_kept=nk, workspace=ws_sel)
        if ev: ev[1].record()
        kv.kv_compact(K, V, kept, nk, seq, out_cap, K_out=Ko, V_out=Vo, pos_out=Po)
        if ev: ev[2].record()

    for _ in range(args.warmup):
        scored_pass()
    torch.cuda.synchronize(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for i in range(args.steps):
        scored_pass(evs[i])
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    k_ms = {name: float(np.mean([evs[i][a].elapsed_time(evs[i][b]) for i in range(args.steps)]))
            for name, a, b in (("tri_score", 0, 1), ("kv_select_topk", 1, 2), ("kv_compact", 2, 3))}
    step_dist = percentiles([evs[i][0].elapsed_time(evs[i][3]) for i in range(args.steps)])
    print(f"[bench] scored pass {ms_step:.3f} ms/step, kernels {k_ms}", file=sys.stderr, flush=True)

    # the same pass captured once into a HIP graph and replayed: the calls only launch kernels on
    # the current stream, so a serving loop can replay them without per-launch host work
    graph_ms = None
    try:
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph):
            scored_pass()
        for _ in range(args.warmup):
            gph.replay()
        torch.cuda.synchronize(dev)
        tg = time.perf_counter()
        for _ in range(args.steps):
            gph.replay()
        torch.cuda.synchronize(dev)
        graph_ms = (time.perf_counter() - tg) * 1e3 / args.steps
        del gph
        print(f"[bench] scored pass replayed from a HIP graph {graph_ms:.3f} ms/step", file=sys.stderr, flush=True)
    except RuntimeError as e:
        print(f"[bench] graph capture unavailable: {e}", file=sys.stderr, flush=True)

    n_kept_head = int(nk[0].item())
    ab = algorithmic_bytes(w, n_kept_head)
    entries = w.entries
    pass_bytes = ab["score"] + ab["select"] + ab["compact"]

    # measured copy ceilings: torch's device copy of a quarter of K, and kv_compact over the
    # contiguous slots 0..n_kept-1 of every head (the pass's compaction bytes, no gather)
    quarter = K[: max(1, L // 4)]
    dst = torch.empty_like(quarter)
    cev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    dst.copy_(quarter)
    cev[0].record()
    for _ in range(args.steps):
        dst.copy_(quarter)
    cev[1].record()
    torch.cuda.synchronize(dev)
    copy_gbs = 2 * quarter.numel() * quarter.element_size() / (cev[0].elapsed_time(cev[1]) / args.steps * 1e-3) / 1e9
    del dst, quarter
    kept_c = torch.arange(b_cap, dtype=torch.int32, device=dev)
    kept_c = torch.where(kept_c < n_kept_head, kept_c, torch.full_like(kept_c, -1)).expand(L, S, H, b_cap).contiguous()
    kv.kv_compact(K, V, kept_c, nk, seq, out_cap, K_out=Ko, V_out=Vo, pos_out=Po)
    cev[0].record()
    for _ in range(args.steps):
        kv.kv_compact(K, V, kept_c, nk, seq, out_cap, K_out=Ko, V_out=Vo, pos_out=Po)
    cev[1].record()
    torch.cuda.synchronize(dev)
    contig_gbs = ab["compact"] / (cev[0].elapsed_time(cev[1]) / args.steps * 1e-3) / 1e9
    del kept_c
    # the score stream's own access pattern with no arithmetic (kv_stream_ceiling over all of K):
    # reads only, and reads plus one 4-byte store per 256 bytes read, as tri_score stores its scores
    k_bytes = K.numel() * K.element_size()
    pat = {}
    if k_bytes % (128 << 10) == 0:
        sink = torch.empty((k_bytes // 256,), dtype=torch.int32, device=dev)
        for tag, stores in (("read", False), ("read_write", True)):
            kv.stream_ceiling(K, sink, stores)
            cev[0].record()
            for _ in range(args.steps):
                kv.stream_ceiling(K, sink, stores)
            cev[1].record()
            torch.cuda.synchronize(dev)
            ms = cev[0].elapsed_time(cev[1]) / args.steps
            moved = k_bytes + (k_bytes // 64 if stores else 0)   # plus 4 bytes per 256 read with stores
            pat[tag] = (ms, moved / (ms * 1e-3) / 1e9)
        del sink
    ceilings = {"device_copy_gbs": copy_gbs, "compact_contiguous_gbs": contig_gbs,
                "kv_compact_frac_of_contiguous": ab["compact"] / (k_ms["kv_compact"] * 1e-3) / 1e9 / contig_gbs,
                "pass_gbs_over_device_copy": pass_bytes / (ms_step * 1e-3) / 1e9 / copy_gbs}
    if pat:
        score_gbs = ab["score"] / (k_ms["tri_score"] * 1e-3) / 1e9
        ceilings.update({"score_pattern_read_gbs": pat["read"][1],
                         "score_pattern_read_write_gbs": pat["read_write"][1],
                         "tri_score_frac_of_pattern": score_gbs / pat["read_write"][1]})
    print(f"[bench] copy ceilings: device copy {copy_gbs:.0f} GB/s, kv_compact on contiguous slots "
          f"{contig_gbs:.0f} GB/s" + (f"; score pattern over K: reads {pat['read'][1]:.0f} GB/s, with stores "
          f"{pat['read_write'][1]:.0f} GB/s ({pat['read_write'][0]:.3f} ms)" if pat else ""),
          file=sys.stderr, flush=True)

    rnd = None
    if not args.no_random:
        for i in range(args.warmup):
            random_pass(i)
        revs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        torch.cuda.synchronize(dev)
        t1 = time.perf_counter()
        for i in range(args.steps):
            random_pass(1000 + i, revs[i])
        torch.cuda.synchronize(dev)
        rwall = (time.perf_counter() - t1) * 1e3 / args.steps
        rk = {"kv_select_random": float(np.mean([revs[i][0].elapsed_time(revs[i][1]) for i in range(args.steps)])),
              "kv_compact": float(np.mean([revs[i][1].elapsed_time(revs[i][2]) for i in range(args.steps)]))}
        rbytes = ab["random_select"] + ab["compact"]
        # the same pass with the draw of layer chunk c + 1 (ALU-bound) running beside the
        # compaction of chunk c (HBM-bound) on a second stream of the same priority; each chunk's
        # call is told its first layer, so the draws, the kept lists and the rows are those of the
        # single call above
        side = torch.cuda.Stream()
        n_chunks = 9   # 4 layers each: measured best of 3-36 chunks (finer ones are bound by the host's launches)
        bounds = np.linspace(0, L, n_chunks + 1).astype(int)
        nks = [torch.empty((S,), dtype=torch.int32, device=dev) for _ in range(n_chunks)]
        cevs = [torch.cuda.Event() for _ in range(n_chunks)]

        def random_pass_overlapped(event):
            cur = torch.cuda.current_stream()
            side.wait_stream(cur)
            for c in range(n_chunks):
                lo, hi = int(bounds[c]), int(bounds[c + 1])
                kv.kv_select_random((hi - lo, S, H, Tc), seq, plen, w.budget, w.recent, w.prompt_cap(),
                                    0x5EED000000000003, event, b_cap=b_cap, kept=kept[lo:hi], n_kept=nks[c],
                                    workspace=ws_sel, layer_base=lo)
                cevs[c].record(cur)
                with torch.cuda.stream(side):
                    side.wait_event(cevs[c])
                    kv.kv_compact(K[lo:hi], V[lo:hi], kept[lo:hi], nks[c], seq, out_cap, K_out=Ko[lo:hi],
                                  V_out=Vo[lo:hi], pos_out=Po[lo:hi])
            cur.wait_stream(side)

        random_pass(4242)
        torch.cuda.synchronize(dev)
        ref_kept, ref_rows = kept.clone(), Ko[:, :, :, :64].clone()
        kept.fill_(-7)
        random_pass_overlapped(4242)
        torch.cuda.synchronize(dev)
        same = bool(torch.equal(kept, ref_kept) and torch.equal(Ko[:, :, :, :64], ref_rows))
        del ref_kept, ref_rows
        for i in range(args.warmup):
            random_pass_overlapped(i)
        torch.cuda.synchronize(dev)
        t2 = time.perf_counter()
        for i in range(args.steps):
            random_pass_overlapped(2000 + i)
        torch.cuda.synchronize(dev)
        owall = (time.perf_counter() - t2) * 1e3 / args.steps
        best = min(rwall, owall)
        rnd = {"ms_per_pass": best, "entries_per_s": entries / (best * 1e-3),
               "gbs": rbytes / (best * 1e-3) / 1e9, "algorithmic_bytes": rbytes,
               "serial": {"ms_per_pass": rwall, "kernel_ms": rk},
               "overlapped": {"ms_per_pass": owall, "layer_chunks": n_chunks, "same_as_serial": same}}
        print(f"[bench] random pass {rwall:.3f} ms serial (kernels {rk}), {owall:.3f} ms with the draw beside the "
              f"compaction in {n_chunks} layer chunks (identical: {same})", file=sys.stderr, flush=True)

    # the full TriAttention score (trigonometric + norm-based term) over the same cache
    from workloads import query_magnitudes
    qabs = torch.from_numpy(query_magnitudes(w, qb)).to(dev)
    for _ in range(args.warmup):
        kv.tri_score(K, qbd, tcur, seq, w.theta, w.deltas, out=scores, qabs=qabs)

    def launches_ms(with_norm):
        fev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        fev[0].record()
        for _ in range(args.steps):
            kv.tri_score(K, qbd, tcur, seq, w.theta, w.deltas, out=scores, qabs=qabs if with_norm else None)
        fev[1].record()
        torch.cuda.synchronize(dev)
        return fev[0].elapsed_time(fev[1]) / args.steps

    # the plain score timed right beside it, alternating, so the ratio compares like with like
    norm_runs, plain_runs = [], []
    for _ in range(2):
        norm_runs.append(launches_ms(True))
        plain_runs.append(launches_ms(False))
    full_ms, plain_ms = min(norm_runs), min(plain_runs)
    norm_ratio = full_ms / plain_ms
    print(f"[bench] tri_score with norm term {full_ms:.3f} ms, plain {plain_ms:.3f} ms beside it "
          f"(ratio {norm_ratio:.3f}{', ABOVE 1.1' if norm_ratio > 1.1 else ''})", file=sys.stderr, flush=True)

    # keys stored after RoPE: dense, and through a block table over the same memory viewed as a
    # paged pool [L, n_blocks, 16, H, d] with a shuffled table
    def time_launches(fn):
        for _ in range(args.warmup):
            fn()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        for _ in range(args.steps):
            fn()
        e[1].record()
        torch.cuda.synchronize(dev)
        return e[0].elapsed_time(e[1]) / args.steps

    rot_ms = time_launches(lambda: kv.tri_score_rotated(K, qbd, tcur, seq, w.theta, w.deltas, out=scores))
    bs = 16
    bps = Tc // bs
    pool = K.view(L, S * bps, bs, H, d)
    gen = torch.Generator(device="cpu")
    gen.manual_seed(7)
    table = torch.randperm(S * bps, generator=gen).view(S, bps).to(torch.int32).to(dev)
    paged_ms = time_launches(lambda: kv.tri_score_rotated(pool, qbd, tcur, seq, w.theta, w.deltas,
                                                          block_table=table, out=scores))
    pool_hm = K.view(L, S * bps, H, bs, d)   # the same bytes as a head-major pool
    paged_hm_ms = time_launches(lambda: kv.tri_score_rotated(pool_hm, qbd, tcur, seq, w.theta, w.deltas,
                                                             block_table=table, out=scores, head_major=True))
    print(f"[bench] rotated keys: dense {rot_ms:.3f} ms, paged {paged_ms:.3f} ms, paged head-major "
          f"{paged_hm_ms:.3f} ms", file=sys.stderr, flush=True)

    # grouped-query scores (z-score per query head, max over the group): the 4 query heads of
    # each KV head of this cache with their own centres, and the gpt-oss-20b-shaped cache
    # (G = 8, head_dim 64) with explicit positions
    from workloads import query_head_centres

    def gqa_case(wg, Kg, seqg, tcurg, posg, keep=False, rotated=None):
        """rotated: None for pre-RoPE keys (tri_score_gqa); else (label, key tensor, block table or None,
        head-major) for the same keys read as stored after RoPE (tri_score_gqa_rotated)."""
        Lg, Sg, Hg, Tg, dg = Kg.shape
        G = wg.group
        # this cache's own query draws are one centre per KV head; the per-query-head centres
        # come from the group-mean recipe with the same shapes
        nud = torch.from_numpy(query_head_centres(wg if wg.q_mode == "group-mean" else
                                                  workload(wg.wid, L=Lg, q_mode="group-mean"))).to(dev)
        outg = torch.empty((Lg, Sg, Hg, Tg), dtype=torch.float32, device=dev)
        head = torch.empty((Lg, Sg, Hg, G, Tg), dtype=torch.float32, device=dev)
        ws = torch.empty((kv.gqa_workspace_bytes(Lg, Sg, Hg, Tg, dg, Kg.dtype, G),), dtype=torch.uint8, device=dev)
        if rotated is None:
            ms = time_launches(lambda: kv.tri_score_gqa(Kg, nud, tcurg, seqg, wg.theta, wg.deltas, pos=posg,
                                                        out=outg, head_out=head, workspace=ws))
        else:
            _, Kr, tab, hm = rotated
            ms = time_launches(lambda: kv.tri_score_gqa_rotated(Kr, nud, tcurg, seqg, wg.theta, wg.deltas,
                                                                block_table=tab, head_major=hm, out=outg,
                                                                head_out=head, workspace=ws))
        n = int(np.sum(np.minimum(wg.seq_len, Tg))) * Lg * Hg
        # each key row read once; G fp32 scores per key written, read back for the z-score, one written
        byts = n * (dg * Kg.element_size() + 8 * G + 4) + (0 if posg is None else n * 4)
        if rotated is not None and rotated[2] is not None:
            byts += rotated[2].numel() * 4 * Lg * Hg      # each (layer, head) reads its sequence's table
        res = {"workload": wg.name, "group": G, "head_dim": dg, "positions": posg is not None,
               "keys": "pre-rope" if rotated is None else rotated[0], "ms_per_launch": ms,
               "entries_per_s": n / (ms * 1e-3), "algorithmic_bytes": byts, "gbs": byts / (ms * 1e-3) / 1e9}
        del ws
        return (res, outg, head) if keep else res

    g3, zmax, head3 = gqa_case(w, K, seq, tcur, None, keep=True)
    gqa = [g3]
    # the same scores over keys stored after RoPE: dense, and the two paged pools above
    gqa_rot = [gqa_case(w, K, seq, tcur, None, rotated=r) for r in
               (("rotated dense", K, None, False), ("rotated paged16", pool, table, False),
                ("rotated paged16 head-major", pool_hm, table, True))]
    print(f"[bench] grouped-query scores over rotated keys: "
          f"{[(g['keys'], round(g['ms_per_launch'], 3)) for g in gqa_rot]}", file=sys.stderr, flush=True)
    # union-based selection over the 4 query heads on those scores (per-head top-k, k = ceil(n_sel/4))
    union_ms = time_launches(lambda: kv.kv_select_union(head3, zmax, seq, plen, w.budget, w.recent, w.prompt_cap(),
                                                        b_cap=b_cap, kept=kept, n_kept=nk))
    union_bytes = entries * 4 * (w.group + 1) + w.n_heads_total * b_cap * 4
    # 131072-token caches (context lengths reach 128K tokens): the same score memory (and the
    # grouped-query scores) viewed as L layers x S/4 seqs x 8 KV heads of 4 * T slots, past the
    # selectors' register tiers
    long_sel = None
    if S % 4 == 0:
        Sl, Tl = S // 4, 4 * Tc
        sc_long = scores.view(L, Sl, H, Tl)
        seq_l, plen_l = i32(np.full(Sl, Tl)), i32(np.full(Sl, w.prompt_len[0]))
        kept_l = torch.empty((L, Sl, H, b_cap), dtype=torch.int32, device=dev)
        nk_l = torch.empty((Sl,), dtype=torch.int32, device=dev)
        lt_ms = time_launches(lambda: kv.kv_select_topk(sc_long, seq_l, plen_l, w.budget, w.recent, w.prompt_cap(),
                                                        b_cap=b_cap, kept=kept_l, n_kept=nk_l))
        lr_ms = time_launches(lambda: kv.kv_select_random((L, Sl, H, Tl), seq_l, plen_l, w.budget, w.recent,
                                                          w.prompt_cap(), 1, 0, b_cap=b_cap, kept=kept_l,
                                                          n_kept=nk_l))
        hs_long, z_long = head3.view(L, Sl, H, w.group, Tl), zmax.view(L, Sl, H, Tl)
        lu_ms = time_launches(lambda: kv.kv_select_union(hs_long, z_long, seq_l, plen_l, w.budget, w.recent,
                                                         w.prompt_cap(), b_cap=b_cap, kept=kept_l, n_kept=nk_l))
        n_long = L * Sl * H * Tl
        long_sel = {"t_cap": Tl, "heads": L * Sl * H, "topk_ms": lt_ms, "random_ms": lr_ms, "union_ms": lu_ms,
                    "topk_entries_per_s": n_long / (lt_ms * 1e-3), "random_entries_per_s": n_long / (lr_ms * 1e-3)}
        print(f"[bench] {Tl}-slot caches: top-k select {lt_ms:.3f} ms, random select {lr_ms:.3f} ms, "
              f"union select {lu_ms:.3f} ms", file=sys.stderr, flush=True)
        del sc_long, kept_l, hs_long, z_long
    del zmax, head3
    recent_ms = time_launches(lambda: kv.kv_select_recent((L, S, H, Tc), seq, plen, w.budget, w.recent,
                                                          w.prompt_cap(), b_cap=b_cap, kept=kept, n_kept=nk))

    w4 = workload(4)
    mu4, qb4, _ = centres(w4)
    K4, _ = kv_torch(w4, dev, mu4, with_values=False)
    pos4 = torch.arange(w4.t_cap, dtype=torch.int32, device=dev).expand(*K4.shape[:4]).contiguous()
    gqa.append(gqa_case(w4, K4, i32(w4.seq_len), i32(w4.t_cur), pos4))
    del K4
    print(f"[bench] grouped-query scores: {[(g['group'], round(g['ms_per_launch'], 3)) for g in gqa]}, "
          f"union select {union_ms:.3f} ms, recency select {recent_ms:.3f} ms", file=sys.stderr, flush=True)

    del pos4
    periodic = periodic_workload(args, dev, time_launches, mu4, qb4)


    cpu = protocol = None
    if timer is not None:
        print(f"[bench] timing the CPU oracle on {timer.cores} worker processes", file=sys.stderr, flush=True)
        protocol = oracle_protocol(timer, dev, args, w, K, V, qb)
        timer.close()
        fp = protocol["full_pass_32k"]["folded"]
        cpu = {"value": fp["entries_per_s"], "unit": "KV entries/s", "cores": timer.cores, "kind": "oracle",
               "host_cpu": cpu_model(), "gpu_over_cpu": entries / (ms_step * 1e-3) / fp["entries_per_s"],
               "sample": f"the whole {w.name} pass ({fp['entries']} entries): folded fp64 score + lexsort top-n "
                         f"select + gather per (layer, seq, KV head), {timer.cores} worker processes, "
                         f"{fp['seconds']:.1f} s; every workload in cpu_protocol"}

    others = None
    if not args.no_other_workloads:
        others = other_workloads(args, dev)

    score_s = k_ms["tri_score"] * 1e-3
    achieved = ab["score"] / score_s / 1e9
    out = {
        "metric": METRIC,
        "value": entries / (ms_step * 1e-3),
        "unit": "KV entries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded concentrated pre-RoPE keys, bf16 K/V resident in HBM)",
        "config": {"workload": w.name, "layers": L, "seqs": S, "kv_heads": H, "head_dim": d, "seq_len": Tc,
                   "prompt": int(w.prompt_len[0]), "budget": w.budget, "recent": w.recent,
                   "rope_theta": w.theta, "n_offsets": len(w.deltas), "kv_dtype": "bf16",
                   "entries_per_pass": entries},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": counter_traffic(), "kernel": "tri_score",
                     "bytes_per_launch": ab["score"], "ms_per_launch": k_ms["tri_score"]},
        "pass": {"algorithmic_bytes": pass_bytes, "gbs": pass_bytes / (ms_step * 1e-3) / 1e9,
                 "frac_of_peak": pass_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                 "step_ms": step_dist,
                 "ceilings": ceilings,
                 "graph_replay_ms": graph_ms,
                 "graph_replay_entries_per_s": None if graph_ms is None else entries / (graph_ms * 1e-3),
                 "kernel_ms": k_ms,
                 "kernel_share": {k: {"bytes": ab[b] / pass_bytes, "time": k_ms[k] / sum(k_ms.values())}
                                  for k, b in (("tri_score", "score"), ("kv_select_topk", "select"),
                                               ("kv_compact", "compact"))},
                 "kernel_gbs": {"tri_score": achieved,
                                "kv_select_topk": ab["select"] / (k_ms["kv_select_topk"] * 1e-3) / 1e9,
                                "kv_compact": ab["compact"] / (k_ms["kv_compact"] * 1e-3) / 1e9}},
        "random_pass": rnd,
        "score_with_norm_term": {"ms_per_launch": full_ms, "gbs": ab["score"] / (full_ms * 1e-3) / 1e9,
                                 "plain_ms_beside": plain_ms, "over_plain": norm_ratio,
                                 "over_plain_above_1_1": norm_ratio > 1.1},
        "score_rotated_keys": {"dense_ms": rot_ms, "dense_gbs": ab["score"] / (rot_ms * 1e-3) / 1e9,
                               "paged16_ms": paged_ms, "paged16_gbs": ab["score"] / (paged_ms * 1e-3) / 1e9,
                               "paged16_head_major_ms": paged_hm_ms,
                               "paged16_head_major_gbs": ab["score"] / (paged_hm_ms * 1e-3) / 1e9},
        "score_gqa": gqa,
        "score_gqa_rotated_keys": gqa_rot,
        "select_union": {"group": w.group, "ms_per_launch": union_ms, "algorithmic_bytes": union_bytes,
                         "gbs": union_bytes / (union_ms * 1e-3) / 1e9},
        "select_recent": {"ms_per_launch": recent_ms},
        "select_long_cache": long_sel,
        "periodic_event": periodic,
        "other_workloads": others,
        "cpu_baseline": cpu,
        "cpu_protocol": protocol,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()

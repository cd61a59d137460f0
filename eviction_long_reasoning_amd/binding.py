"""Torch-tensor front end of the C ABI (argument marshalling only).

Each function checks devices, dtypes and shapes, allocates outputs that were
not supplied, and passes raw device pointers plus torch's current HIP stream
to the library. All arithmetic happens in the HIP kernels.

Tensor layouts (head-major, see include/kvevict.h):
  K, V        [L, S, H, t_cap, d]  float32 or bfloat16
  pos         [L, S, H, t_cap]     int32 (optional; slot index otherwise)
  qbar        [L, H, d]            float32
  scores      [L, S, H, t_cap]     float32
  kept        [L, S, H, b_cap]     int32
  seq_len, prompt_len, t_cur, n_kept  [S] int32
  workspace   uint8 GPU tensor of at least the matching *_workspace_bytes query (allocated per
              call when omitted; pass one to keep calls allocation-free)
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import torch

from . import _lib

_DT = {torch.float32: _lib.KV_F32, torch.bfloat16: _lib.KV_BF16}


def _dev_ptr(t: Optional[torch.Tensor], name: str, dtype=None, shape=None, device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return ctypes.c_void_p(t.data_ptr())


def _invoke(name: str, device, *args) -> None:
    """Call entry point ``name`` with ``device`` current and its current stream as the last argument.

    The library launches on the calling thread's current HIP device, so a tensor on another device
    than the current one would otherwise get its kernels on the wrong GPU.
    """
    fn = getattr(_lib.load(), name)
    with torch.cuda.device(device):
        st = fn(*args, ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream))
    _lib.check(name, st)


def _shape(L, S, H, d, t_cap, dtype_code, seq_len_ptr) -> _lib.KvShape:
    return _lib.KvShape(int(L), int(S), int(H), int(d), int(t_cap), int(dtype_code), seq_len_ptr)


def _workspace(ws: Optional[torch.Tensor], need: int, device):
    """(tensor, pointer, bytes) of the caller's workspace, or of a fresh one of ``need`` bytes."""
    if ws is None:
        ws = torch.empty((max(int(need), _lib.KV_WORKSPACE_HEADER),), dtype=torch.uint8, device=device)
    return ws, _dev_ptr(ws, "workspace", torch.uint8, None, device), ws.numel()


def score_workspace_bytes(L: int, S: int, H: int, t_cap: int, d: int, dtype: torch.dtype, n_delta: int) -> int:
    """Workspace bytes ``tri_score`` needs (0 for a shape or offset count it rejects)."""
    shape = _shape(L, S, H, d, t_cap, _DT[dtype], None)
    return int(_lib.load().kv_score_workspace_bytes(ctypes.byref(shape), int(n_delta)))


def select_workspace_bytes(L: int, S: int, H: int, t_cap: int, b_cap: int) -> int:
    """Workspace bytes ``kv_select_topk`` / ``kv_select_random(_shared)`` need (0 if rejected)."""
    shape = _shape(L, S, H, 0, t_cap, 0, None)
    return int(_lib.load().kv_select_workspace_bytes(ctypes.byref(shape), int(b_cap)))


def tri_score(K: torch.Tensor, qbar: torch.Tensor, t_cur: torch.Tensor, seq_len: torch.Tensor,
              rope_theta: float, deltas: Sequence[int], pos: Optional[torch.Tensor] = None,
              out: Optional[torch.Tensor] = None, qabs: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Offset-averaged RoPE query-centre score of every cached key (fp32 [L,S,H,t_cap]).

    With ``qabs`` ([L,H,d/2] fp32, mean query magnitude per band) the norm-based term is added.
    """
    if K.dim() != 5 or K.dtype not in _DT:
        raise ValueError("K must be [L,S,H,t_cap,d] float32/bfloat16")
    L, S, H, t_cap, d = K.shape
    dev = K.device
    kp = _dev_ptr(K, "K")
    qp = _dev_ptr(qbar, "qbar", torch.float32, (L, H, d), dev)
    tp = _dev_ptr(t_cur, "t_cur", torch.int32, (S,), dev)
    sp = _dev_ptr(seq_len, "seq_len", torch.int32, (S,), dev)
    pp = _dev_ptr(pos, "pos", torch.int32, (L, S, H, t_cap), dev)
    ap = _dev_ptr(qabs, "qabs", torch.float32, (L, H, d // 2), dev)
    if out is None:
        out = torch.empty((L, S, H, t_cap), dtype=torch.float32, device=dev)
    op = _dev_ptr(out, "out", torch.float32, (L, S, H, t_cap), dev)
    dl = [int(x) for x in deltas]
    arr = (ctypes.c_int32 * max(1, len(dl)))(*dl)
    shape = _shape(L, S, H, d, t_cap, _DT[K.dtype], sp)
    need = int(_lib.load().kv_score_workspace_bytes(ctypes.byref(shape), len(dl)))
    workspace, wp, wb = _workspace(workspace, need, dev)
    _invoke("tri_score", dev, ctypes.byref(shape), kp, pp, qp, ap, tp, float(rope_theta), arr, len(dl), op, wp, wb)
    return out


def tri_score_rotated(K: torch.Tensor, qbar: torch.Tensor, t_cur: torch.Tensor, seq_len: torch.Tensor,
                      rope_theta: float, deltas: Sequence[int], rope_style: str = "interleaved",
                      block_table: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                      qabs: Optional[torch.Tensor] = None, head_major: bool = False) -> torch.Tensor:
    """Scores of keys stored after RoPE (fp32 [L,S,H,t_cap]).

    Dense: ``K`` is [L,S,H,t_cap,d]. Paged: ``K`` is the pool [L,n_blocks,block_size,H,d]
    ([L,n_blocks,H,block_size,d] with ``head_major``) and ``block_table`` is int32
    [S, blocks_per_seq]; t_cap = blocks_per_seq * block_size.
    ``rope_style`` is "interleaved" (x[2f], x[2f+1]) or "half" (x[f], x[f+d/2]).
    """
    if K.dim() != 5 or K.dtype not in _DT:
        raise ValueError("K must be a 5-D float32/bfloat16 tensor")
    style = {"interleaved": _lib.KV_ROPE_INTERLEAVED, "half": _lib.KV_ROPE_HALF}[rope_style]
    dev = K.device
    paged = None
    if block_table is None:
        L, S, H, t_cap, d = K.shape
    else:
        if head_major:
            L, n_blocks, H, bs, d = K.shape
        else:
            L, n_blocks, bs, H, d = K.shape
        S, bps = block_table.shape
        t_cap = bps * bs
        paged = _lib.KvPaged(_dev_ptr(block_table, "block_table", torch.int32, (S, bps), dev), int(bps), int(bs),
                             int(n_blocks), int(bool(head_major)))
    kp = _dev_ptr(K, "K")
    qp = _dev_ptr(qbar, "qbar", torch.float32, (L, H, d), dev)
    ap = _dev_ptr(qabs, "qabs", torch.float32, (L, H, d // 2), dev)
    tp = _dev_ptr(t_cur, "t_cur", torch.int32, (S,), dev)
    sp = _dev_ptr(seq_len, "seq_len", torch.int32, (S,), dev)
    if out is None:
        out = torch.empty((L, S, H, t_cap), dtype=torch.float32, device=dev)
    op = _dev_ptr(out, "out", torch.float32, (L, S, H, t_cap), dev)
    dl = [int(x) for x in deltas]
    arr = (ctypes.c_int32 * max(1, len(dl)))(*dl)
    shape = _shape(L, S, H, d, t_cap, _DT[K.dtype], sp)
    _invoke("tri_score_rotated", dev, ctypes.byref(shape), kp, None if paged is None else ctypes.byref(paged),
            style, qp, ap, tp, float(rope_theta), arr, len(dl), op)
    return out


def tri_score_gqa(K: torch.Tensor, qbar: torch.Tensor, t_cur: torch.Tensor, seq_len: torch.Tensor,
                  rope_theta: float, deltas: Sequence[int], pos: Optional[torch.Tensor] = None,
                  qabs: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                  head_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None
                  ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Grouped-query scores: (max over the group of the z-normalised per-query-head scores
    [L,S,H,t_cap], the per-query-head scores [L,S,H,G,t_cap]).

    ``qbar`` is [L,H,G,d] fp32 (one centre per query head), ``qabs`` optionally [L,H,G,d/2].
    ``workspace`` is a uint8 GPU tensor of at least ``gqa_workspace_bytes`` bytes (allocated
    here when omitted).
    """
    if K.dim() != 5 or K.dtype not in _DT:
        raise ValueError("K must be [L,S,H,t_cap,d] float32/bfloat16")
    if qbar.dim() != 4:
        raise ValueError("qbar must be [L,H,G,d]")
    L, S, H, t_cap, d = K.shape
    G = qbar.shape[2]
    dev = K.device
    kp = _dev_ptr(K, "K")
    qp = _dev_ptr(qbar, "qbar", torch.float32, (L, H, G, d), dev)
    tp = _dev_ptr(t_cur, "t_cur", torch.int32, (S,), dev)
    sp = _dev_ptr(seq_len, "seq_len", torch.int32, (S,), dev)
    pp = _dev_ptr(pos, "pos", torch.int32, (L, S, H, t_cap), dev)
    ap = _dev_ptr(qabs, "qabs", torch.float32, (L, H, G, d // 2), dev)
    if out is None:
        out = torch.empty((L, S, H, t_cap), dtype=torch.float32, device=dev)
    if head_out is None:
        head_out = torch.empty((L, S, H, G, t_cap), dtype=torch.float32, device=dev)
    op = _dev_ptr(out, "out", torch.float32, (L, S, H, t_cap), dev)
    hp = _dev_ptr(head_out, "head_out", torch.float32, (L, S, H, G, t_cap), dev)
    shape = _shape(L, S, H, d, t_cap, _DT[K.dtype], sp)
    need = int(_lib.load().kv_score_gqa_workspace_bytes(ctypes.byref(shape), int(G)))
    workspace, wp, _ = _workspace(workspace, need, dev)
    dl = [int(x) for x in deltas]
    arr = (ctypes.c_int32 * max(1, len(dl)))(*dl)
    _invoke("tri_score_gqa", dev, ctypes.byref(shape), kp, pp, int(G), qp, ap, tp, float(rope_theta), arr,
            len(dl), hp, op, wp, workspace.numel())
    return out, head_out


def tri_score_gqa_noalloc(K: torch.Tensor, qbar: torch.Tensor, t_cur: torch.Tensor, seq_len: torch.Tensor,
                          rope_theta: float, deltas: Sequence[int], out: torch.Tensor, head_out: torch.Tensor,
                          pos: Optional[torch.Tensor] = None, qabs: Optional[torch.Tensor] = None) -> None:
    """``tri_score_gqa`` without a workspace: the library's own device array holds the partial sums
    and nothing is allocated (``out`` and ``head_out`` are required). Calls on one device must not
    overlap in time."""
    if K.dim() != 5 or K.dtype not in _DT or qbar.dim() != 4:
        raise ValueError("K must be [L,S,H,t_cap,d] float32/bfloat16 and qbar [L,H,G,d]")
    L, S, H, t_cap, d = K.shape
    G = qbar.shape[2]
    dev = K.device
    kp = _dev_ptr(K, "K")
    qp = _dev_ptr(qbar, "qbar", torch.float32, (L, H, G, d), dev)
    tp = _dev_ptr(t_cur, "t_cur", torch.int32, (S,), dev)
    sp = _dev_ptr(seq_len, "seq_len", torch.int32, (S,), dev)
    pp = _dev_ptr(pos, "pos", torch.int32, (L, S, H, t_cap), dev)
    ap = _dev_ptr(qabs, "qabs", torch.float32, (L, H, G, d // 2), dev)
    op = _dev_ptr(out, "out", torch.float32, (L, S, H, t_cap), dev)
    hp = _dev_ptr(head_out, "head_out", torch.float32, (L, S, H, G, t_cap), dev)
    shape = _shape(L, S, H, d, t_cap, _DT[K.dtype], sp)
    dl = [int(x) for x in deltas]
    arr = (ctypes.c_int32 * max(1, len(dl)))(*dl)
    _invoke("tri_score_gqa_noalloc", dev, ctypes.byref(shape), kp, pp, int(G), qp, ap, tp, float(rope_theta), arr,
            len(dl), hp, op)


def tri_score_gqa_rotated(K: torch.Tensor, qbar: torch.Tensor, t_cur: torch.Tensor, seq_len: torch.Tensor,
                          rope_theta: float, deltas: Sequence[int], rope_style: str = "interleaved",
                          block_table: Optional[torch.Tensor] = None, head_major: bool = False,
                          qabs: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                          head_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None
                          ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Grouped-query scores of keys stored after RoPE: (max over the group of the z-normalised
    per-query-head scores [L,S,H,t_cap], the per-query-head scores [L,S,H,G,t_cap]).

    ``K`` and ``block_table`` as for ``tri_score_rotated``; ``qbar`` is [L,H,G,d] fp32 and ``qabs``
    optionally [L,H,G,d/2], both in the stored keys' pairing.
    """
    if K.dim() != 5 or K.dtype not in _DT:
        raise ValueError("K must be a 5-D float32/bfloat16 tensor")
    if qbar.dim() != 4:
        raise ValueError("qbar must be [L,H,G,d]")
    style = {"interleaved": _lib.KV_ROPE_INTERLEAVED, "half": _lib.KV_ROPE_HALF}[rope_style]
    dev = K.device
    paged = None
    if block_table is None:
        L, S, H, t_cap, d = K.shape
    else:
        if head_major:
            L, n_blocks, H, bs, d = K.shape
        else:
            L, n_blocks, bs, H, d = K.shape
        S, bps = block_table.shape
        t_cap = bps * bs
        paged = _lib.KvPaged(_dev_ptr(block_table, "block_table", torch.int32, (S, bps), dev), int(bps), int(bs),
                             int(n_blocks), int(bool(head_major)))
    G = qbar.shape[2]
    kp = _dev_ptr(K, "K")
    qp = _dev_ptr(qbar, "qbar", torch.float32, (L, H, G, d), dev)
    ap = _dev_ptr(qabs, "qabs", torch.float32, (L, H, G, d // 2), dev)
    tp = _dev_ptr(t_cur, "t_cur", torch.int32, (S,), dev)
    sp = _dev_ptr(seq_len, "seq_len", torch.int32, (S,), dev)
    if out is None:
        out = torch.empty((L, S, H, t_cap), dtype=torch.float32, device=dev)
    if head_out is None:
        head_out = torch.empty((L, S, H, G, t_cap), dtype=torch.float32, device=dev)
    op = _dev_ptr(out, "out", torch.float32, (L, S, H, t_cap), dev)
    hp = _dev_ptr(head_out, "head_out", torch.float32, (L, S, H, G, t_cap), dev)
    shape = _shape(L, S, H, d, t_cap, _DT[K.dtype], sp)
    need = int(_lib.load().kv_score_gqa_workspace_bytes(ctypes.byref(shape), int(G)))
    workspace, wp, _ = _workspace(workspace, need, dev)
    dl = [int(x) for x in deltas]
    arr = (ctypes.c_int32 * max(1, len(dl)))(*dl)
    _invoke("tri_score_gqa_rotated", dev, ctypes.byref(shape), kp, None if paged is None else ctypes.byref(paged),
            style, int(G), qp, ap, tp, float(rope_theta), arr, len(dl), hp, op, wp, workspace.numel())
    return out, head_out


def gqa_workspace_bytes(L: int, S: int, H: int, t_cap: int, d: int, dtype: torch.dtype, group: int) -> int:
    """Workspace bytes ``tri_score_gqa`` needs (0 for a shape or group it rejects)."""
    shape = _shape(L, S, H, d, t_cap, _DT[dtype], None)
    return int(_lib.load().kv_score_gqa_workspace_bytes(ctypes.byref(shape), int(group)))


def _select_io(L, S, H, b_cap, device, kept, n_kept):
    if kept is None:
        kept = torch.empty((L, S, H, b_cap), dtype=torch.int32, device=device)
    if n_kept is None:
        n_kept = torch.empty((S,), dtype=torch.int32, device=device)
    kp = _dev_ptr(kept, "kept", torch.int32, (L, S, H, b_cap), device)
    np_ = _dev_ptr(n_kept, "n_kept", torch.int32, (S,), device)
    return kept, n_kept, kp, np_


def kv_select_topk(scores: torch.Tensor, seq_len: torch.Tensor, prompt_len: torch.Tensor, budget: int,
                   recent: int, prompt_cap: int, b_cap: Optional[int] = None,
                   kept: Optional[torch.Tensor] = None, n_kept: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-head kept slots (ascending, -1 padded) under the top-n rule, and n_kept per sequence."""
    if scores.dim() != 4:
        raise ValueError("scores must be [L,S,H,t_cap]")
    L, S, H, t_cap = scores.shape
    dev = scores.device
    b_cap = int(b_cap if b_cap is not None else max(budget, prompt_cap))
    sc = _dev_ptr(scores, "scores", torch.float32)
    sp = _dev_ptr(seq_len, "seq_len", torch.int32, (S,), dev)
    pl = _dev_ptr(prompt_len, "prompt_len", torch.int32, (S,), dev)
    kept, n_kept, kp, nkp = _select_io(L, S, H, b_cap, dev, kept, n_kept)
    shape = _shape(L, S, H, 0, t_cap, 0, sp)
    pol = _lib.KvPolicy(int(budget), int(recent), int(prompt_cap), pl)
    need = int(_lib.load().kv_select_workspace_bytes(ctypes.byref(shape), b_cap))
    workspace, wp, wb = _workspace(workspace, need, dev)
    _invoke("kv_select_topk", dev, ctypes.byref(shape), ctypes.byref(pol), sc, kp, b_cap, nkp, wp, wb)
    return kept, n_kept


def kv_select_random(cache_shape: Tuple[int, int, int, int], seq_len: torch.Tensor, prompt_len: torch.Tensor,
                     budget: int, recent: int, prompt_cap: int, seed: int, event: int,
                     pos: Optional[torch.Tensor] = None, b_cap: Optional[int] = None,
                     kept: Optional[torch.Tensor] = None, n_kept: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, layer_base: int = 0
                     ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-head kept slots under Random Attention's rule (Philox draw per head and event).

    ``layer_base`` is the model index of the first layer of ``cache_shape`` (layer l draws as layer
    layer_base + l), so a pass split into layer chunks draws what one call over all layers draws."""
    L, S, H, t_cap = (int(x) for x in cache_shape)
    dev = seq_len.device
    b_cap = int(b_cap if b_cap is not None else max(budget, prompt_cap))
    sp = _dev_ptr(seq_len, "seq_len", torch.int32, (S,), dev)
    pl = _dev_ptr(prompt_len, "prompt_len", torch.int32, (S,), dev)
    pp = _dev_ptr(pos, "pos", torch.int32, (L, S, H, t_cap), dev)
    kept, n_kept, kp, nkp = _select_io(L, S, H, b_cap, dev, kept, n_kept)
    shape = _shape(L, S, H, 0, t_cap, 0, sp)
    pol = _lib.KvPolicy(int(budget), int(recent), int(prompt_cap), pl)
    need = int(_lib.load().kv_select_workspace_bytes(ctypes.byref(shape), b_cap))
    workspace, wp, wb = _workspace(workspace, need, dev)
    _invoke("kv_select_random", dev, ctypes.byref(shape), ctypes.byref(pol), pp, int(seed) & (2 ** 64 - 1),
            int(event) & 0xFFFFFFFF, int(layer_base), kp, b_cap, nkp, wp, wb)
    return kept, n_kept


def kv_select_union(head_scores: torch.Tensor, scores: torch.Tensor, seq_len: torch.Tensor,
                    prompt_len: torch.Tensor, budget: int, recent: int, prompt_cap: int, k_per_head: int = 0,
                    b_cap: Optional[int] = None, kept: Optional[torch.Tensor] = None,
                    n_kept: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Union of the per-query-head top-k sets, final choice by the combined score.

    ``head_scores`` is [L,S,H,G,t_cap] and ``scores`` (the combined score) [L,S,H,t_cap], both
    fp32, as ``tri_score_gqa`` returns them; ``k_per_head`` <= 0 means ceil(n_sel / G).
    """
    if head_scores.dim() != 5 or scores.dim() != 4:
        raise ValueError("head_scores must be [L,S,H,G,t_cap] and scores [L,S,H,t_cap]")
    L, S, H, G, t_cap = head_scores.shape
    dev = scores.device
    b_cap = int(b_cap if b_cap is not None else max(budget, prompt_cap))
    hp = _dev_ptr(head_scores, "head_scores", torch.float32, (L, S, H, G, t_cap), dev)
    cp = _dev_ptr(scores, "scores", torch.float32, (L, S, H, t_cap), dev)
    sp = _dev_ptr(seq_len, "seq_len", torch.int32, (S,), dev)
    pl = _dev_ptr(prompt_len, "prompt_len", torch.int32, (S,), dev)
    kept, n_kept, kp, nkp = _select_io(L, S, H, b_cap, dev, kept, n_kept)
    shape = _shape(L, S, H, 0, t_cap, 0, sp)
    pol = _lib.KvPolicy(int(budget), int(recent), int(prompt_cap), pl)
    _invoke("kv_select_union", dev, ctypes.byref(shape), ctypes.byref(pol), int(G), int(k_per_head), hp, cp, kp,
            b_cap, nkp)
    return kept, n_kept


def kv_select_random_shared(cache_shape: Tuple[int, int, int, int], seq_len: torch.Tensor,
                            prompt_len: torch.Tensor, budget: int, recent: int, prompt_cap: int, seed: int,
                            event: int, pos: Optional[torch.Tensor] = None, b_cap: Optional[int] = None,
                            kept: Optional[torch.Tensor] = None, n_kept: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """The shared-draw control: every head keeps what layer 0 / KV head 0 would draw."""
    L, S, H, t_cap = (int(x) for x in cache_shape)
    dev = seq_len.device
    b_cap = int(b_cap if b_cap is not None else max(budget, prompt_cap))
    sp = _dev_ptr(seq_len, "seq_len", torch.int32, (S,), dev)
    pl = _dev_ptr(prompt_len, "prompt_len", torch.int32, (S,), dev)
    pp = _dev_ptr(pos, "pos", torch.int32, (L, S, H, t_cap), dev)
    kept, n_kept, kp, nkp = _select_io(L, S, H, b_cap, dev, kept, n_kept)
    shape = _shape(L, S, H, 0, t_cap, 0, sp)
    pol = _lib.KvPolicy(int(budget), int(recent), int(prompt_cap), pl)
    need = int(_lib.load().kv_select_workspace_bytes(ctypes.byref(shape), b_cap))
    workspace, wp, wb = _workspace(workspace, need, dev)
    _invoke("kv_select_random_shared", dev, ctypes.byref(shape), ctypes.byref(pol), pp,
            int(seed) & (2 ** 64 - 1), int(event) & 0xFFFFFFFF, kp, b_cap, nkp, wp, wb)
    return kept, n_kept


def kv_select_recent(cache_shape: Tuple[int, int, int, int], seq_len: torch.Tensor, prompt_len: torch.Tensor,
                     budget: int, recent: int, prompt_cap: int, b_cap: Optional[int] = None,
                     kept: Optional[torch.Tensor] = None, n_kept: Optional[torch.Tensor] = None
                     ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Recency+prompt: the prompt and the latest slots of each head (no scores)."""
    L, S, H, t_cap = (int(x) for x in cache_shape)
    dev = seq_len.device
    b_cap = int(b_cap if b_cap is not None else max(budget, prompt_cap))
    sp = _dev_ptr(seq_len, "seq_len", torch.int32, (S,), dev)
    pl = _dev_ptr(prompt_len, "prompt_len", torch.int32, (S,), dev)
    kept, n_kept, kp, nkp = _select_io(L, S, H, b_cap, dev, kept, n_kept)
    shape = _shape(L, S, H, 0, t_cap, 0, sp)
    pol = _lib.KvPolicy(int(budget), int(recent), int(prompt_cap), pl)
    _invoke("kv_select_recent", dev, ctypes.byref(shape), ctypes.byref(pol), kp, b_cap, nkp)
    return kept, n_kept


def kv_audit_kept(kept: torch.Tensor, n_kept: torch.Tensor, seq_len: torch.Tensor, prompt_len: torch.Tensor,
                  budget: int, recent: int, prompt_cap: int, t_cap: int,
                  bad: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-head count of kept-list entries that break the partition rules (int32 [L,S,H]; 0 = valid)."""
    if kept.dim() != 4:
        raise ValueError("kept must be [L,S,H,b_cap]")
    L, S, H, b_cap = kept.shape
    dev = kept.device
    kp = _dev_ptr(kept, "kept", torch.int32, (L, S, H, b_cap), dev)
    nkp = _dev_ptr(n_kept, "n_kept", torch.int32, (S,), dev)
    sp = _dev_ptr(seq_len, "seq_len", torch.int32, (S,), dev)
    pl = _dev_ptr(prompt_len, "prompt_len", torch.int32, (S,), dev)
    if bad is None:
        bad = torch.empty((L, S, H), dtype=torch.int32, device=dev)
    bp = _dev_ptr(bad, "bad", torch.int32, (L, S, H), dev)
    shape = _shape(L, S, H, 0, int(t_cap), 0, sp)
    pol = _lib.KvPolicy(int(budget), int(recent), int(prompt_cap), pl)
    _invoke("kv_audit_kept", dev, ctypes.byref(shape), ctypes.byref(pol), kp, int(b_cap), nkp, bp)
    return bad


def stream_ceiling(buf: torch.Tensor, out: torch.Tensor, with_stores: bool) -> None:
    """Measurement aid: read ``buf`` (a contiguous GPU tensor of a whole number of 128 KB) with
    tri_score's access pattern and no arithmetic, writing one 4-byte value per 256 bytes read into
    ``out`` (with_stores) or one per 32 KB (without). See kv_stream_ceiling in include/kvevict.h."""
    dev = buf.device
    bp = _dev_ptr(buf, "buf", None, None, dev)
    nbytes = buf.numel() * buf.element_size()
    need = nbytes // 256 if with_stores else nbytes // 32768
    op = _dev_ptr(out, "out", None, None, dev)
    if out.numel() * out.element_size() < 4 * need:
        raise ValueError(f"out must hold {need} 4-byte words")
    _invoke("kv_stream_ceiling", dev, bp, ctypes.c_size_t(nbytes), op, int(bool(with_stores)))


def kv_compact_inplace(K: torch.Tensor, V: torch.Tensor, kept: torch.Tensor, n_kept: torch.Tensor,
                       seq_len: torch.Tensor, pos: Optional[torch.Tensor] = None) -> None:
    """In-place hole filling: afterwards slots 0..n_kept-1 of each head hold the kept rows."""
    if K.dim() != 5 or K.dtype not in _DT or V.shape != K.shape or V.dtype != K.dtype:
        raise ValueError("K and V must both be [L,S,H,t_cap,d] of the same float32/bfloat16 dtype")
    L, S, H, t_cap, d = K.shape
    dev = K.device
    b_cap = kept.shape[-1]
    kp_, vp_ = _dev_ptr(K, "K"), _dev_ptr(V, "V", None, None, dev)
    kp = _dev_ptr(kept, "kept", torch.int32, (L, S, H, b_cap), dev)
    nkp = _dev_ptr(n_kept, "n_kept", torch.int32, (S,), dev)
    sp = _dev_ptr(seq_len, "seq_len", torch.int32, (S,), dev)
    pp = _dev_ptr(pos, "pos", torch.int32, (L, S, H, t_cap), dev)
    shape = _shape(L, S, H, d, t_cap, _DT[K.dtype], sp)
    _invoke("kv_compact_inplace", dev, ctypes.byref(shape), kp_, vp_, pp, kp, int(b_cap), nkp)


def kv_compact(K: torch.Tensor, V: torch.Tensor, kept: torch.Tensor, n_kept: torch.Tensor, seq_len: torch.Tensor,
               out_cap: int, pos: Optional[torch.Tensor] = None, with_pos: bool = True,
               K_out: Optional[torch.Tensor] = None, V_out: Optional[torch.Tensor] = None,
               pos_out: Optional[torch.Tensor] = None):
    """Gather kept rows: returns (K_out, V_out, pos_out) shaped [L,S,H,out_cap,(d)]."""
    if K.dim() != 5 or K.dtype not in _DT or V.shape != K.shape or V.dtype != K.dtype:
        raise ValueError("K and V must both be [L,S,H,t_cap,d] of the same float32/bfloat16 dtype")
    L, S, H, t_cap, d = K.shape
    dev = K.device
    b_cap = kept.shape[-1]
    kin, vin = _dev_ptr(K, "K"), _dev_ptr(V, "V", None, None, dev)
    kp = _dev_ptr(kept, "kept", torch.int32, (L, S, H, b_cap), dev)
    nkp = _dev_ptr(n_kept, "n_kept", torch.int32, (S,), dev)
    sp = _dev_ptr(seq_len, "seq_len", torch.int32, (S,), dev)
    pp = _dev_ptr(pos, "pos", torch.int32, (L, S, H, t_cap), dev)
    if K_out is None:
        K_out = torch.empty((L, S, H, out_cap, d), dtype=K.dtype, device=dev)
    if V_out is None:
        V_out = torch.empty((L, S, H, out_cap, d), dtype=K.dtype, device=dev)
    if with_pos and pos_out is None:
        pos_out = torch.empty((L, S, H, out_cap), dtype=torch.int32, device=dev)
    kop = _dev_ptr(K_out, "K_out", K.dtype, (L, S, H, out_cap, d), dev)
    vop = _dev_ptr(V_out, "V_out", K.dtype, (L, S, H, out_cap, d), dev)
    pop = _dev_ptr(pos_out, "pos_out", torch.int32, (L, S, H, out_cap), dev)
    shape = _shape(L, S, H, d, t_cap, _DT[K.dtype], sp)
    _invoke("kv_compact", dev, ctypes.byref(shape), kin, vin, pp, kp, int(b_cap), nkp, kop, vop, pop,
            int(out_cap))
    return K_out, V_out, pos_out

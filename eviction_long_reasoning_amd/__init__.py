"""MI355X-native KV-cache eviction hot path: score, select, compact.

The four operations of one eviction pass are hand-written HIP kernels for
gfx950 behind a C ABI (``include/kvevict.h``, ``libkvevict.so``); this
package is a thin torch-tensor binding over it.

  tri_score         offset-averaged RoPE query-centre score of every key
  tri_score_rotated the same for keys stored after RoPE, dense or paged
  tri_score_gqa     per-query-head scores of a GQA group, z-normalised, max over the group
  tri_score_gqa_rotated  the same for keys stored after RoPE, dense or paged
  tri_score_gqa_noalloc  tri_score_gqa with the library's own scratch array (allocates nothing)
  kv_select_topk    keep prompt + recent window + top-scoring keys per head
  kv_select_random  keep prompt + recent window + per-head uniform random keys
  kv_compact        gather kept K/V rows and positions contiguously

and the policy variants:

  kv_select_union          union of per-query-head top-k sets, ranked by a combined score
  kv_select_random_shared  one random keep-set shared by every head
  kv_select_recent         keep the prompt and the latest slots
  kv_compact_inplace       fill evicted slots with the kept rows beyond the new length
  kv_audit_kept            per-head count of kept-list entries that break the partition rules

and a measurement aid:

  stream_ceiling           tri_score's loads (and stores) without its arithmetic

The binding holds no arithmetic of its own and has no CPU fallback: without
the built library every call raises.
"""
from ._lib import KvError, library_path, load as load_library
from .binding import (gqa_workspace_bytes, kv_audit_kept, kv_compact, kv_compact_inplace, kv_select_random,
                      kv_select_random_shared, kv_select_recent, kv_select_union, kv_select_topk,
                      score_workspace_bytes, select_workspace_bytes, stream_ceiling, tri_score, tri_score_gqa,
                      tri_score_gqa_noalloc, tri_score_gqa_rotated, tri_score_rotated)

__all__ = ["tri_score", "tri_score_rotated", "tri_score_gqa", "tri_score_gqa_rotated", "tri_score_gqa_noalloc",
           "gqa_workspace_bytes",
           "score_workspace_bytes", "select_workspace_bytes", "kv_select_topk", "kv_select_random", "kv_compact",
           "kv_select_union", "kv_select_random_shared", "kv_select_recent", "kv_compact_inplace", "kv_audit_kept",
           "stream_ceiling",
           "KvError", "library_path", "load_library"]

// Host-side argument checks of the C ABI, run under AddressSanitizer (CPU only).
//
// Every call below is rejected on the host before any HIP call, so no GPU is needed; the
// sanitizer watches the validation code (shape arithmetic, overlap tests, workspace sizing)
// for out-of-bounds or use-after-free accesses. Exit status 0 means every expected status came
// back and the sanitizer stayed silent.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "kvevict.h"

static int failures = 0;
#define EXPECT(call, want)                                                             \
  do {                                                                                 \
    const int got_ = static_cast<int>(call);                                           \
    if (got_ != (want)) {                                                              \
      std::fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, \
                   static_cast<int>(want));                                           \
      ++failures;                                                                      \
    }                                                                                  \
  } while (0)

int main() {
  void *dummy = reinterpret_cast<void *>(0x1000);
  const int32_t *seq = reinterpret_cast<const int32_t *>(0x2000);
  int32_t deltas[3] = {1, 2, 4};
  kv_shape sh{1, 1, 1, 128, 4096, KV_BF16, seq};
  kv_policy pol{1024, 64, 128, seq};

  if (kv_version() >> 16 != 2) ++failures;
  if (kv_device_checks() != 0) ++failures;
  void *wsp = reinterpret_cast<void *>(0x7000000);
  for (int s = -6; s <= 1; ++s)
    if (!kv_status_string(s) || !std::strlen(kv_status_string(s))) ++failures;

  // scoring: null shape, bad head_dim, bad dtype, misaligned keys, no offsets, bad theta
  EXPECT(tri_score(nullptr, dummy, nullptr, (const float *)dummy, nullptr, seq, 1e4, deltas, 3, (float *)dummy, wsp, 1 << 20, nullptr), KV_EINVAL);
  kv_shape odd = sh;
  odd.head_dim = 7;
  EXPECT(tri_score(&odd, dummy, nullptr, (const float *)dummy, nullptr, seq, 1e4, deltas, 3, (float *)dummy, wsp, 1 << 20, nullptr), KV_ESHAPE);
  kv_shape bad_dtype = sh;
  bad_dtype.dtype = 9;
  EXPECT(tri_score(&bad_dtype, dummy, nullptr, (const float *)dummy, nullptr, seq, 1e4, deltas, 3, (float *)dummy, wsp, 1 << 20, nullptr), KV_EDTYPE);
  EXPECT(tri_score(&sh, (void *)0x1008, nullptr, (const float *)dummy, nullptr, seq, 1e4, deltas, 3, (float *)dummy, wsp, 1 << 20, nullptr), KV_EINVAL);
  EXPECT(tri_score(&sh, dummy, nullptr, (const float *)dummy, nullptr, seq, 1e4, deltas, 0, (float *)dummy, wsp, 1 << 20, nullptr), KV_EINVAL);
  EXPECT(tri_score(&sh, dummy, nullptr, (const float *)dummy, nullptr, seq, -1.0, deltas, 3, (float *)dummy, wsp, 1 << 20, nullptr), KV_EINVAL);

  // rotated keys: unknown style and pool layout, a block table too short for t_cap
  EXPECT(tri_score_rotated(&sh, dummy, nullptr, 7, (const float *)dummy, nullptr, seq, 1e4, deltas, 3, (float *)dummy, nullptr), KV_EINVAL);
  kv_paged pg{seq, 4, 16, 8, 2};
  EXPECT(tri_score_rotated(&sh, dummy, &pg, 0, (const float *)dummy, nullptr, seq, 1e4, deltas, 3, (float *)dummy, nullptr), KV_EINVAL);
  pg.head_major = 1;
  EXPECT(tri_score_rotated(&sh, dummy, &pg, 0, (const float *)dummy, nullptr, seq, 1e4, deltas, 3, (float *)dummy, nullptr), KV_ESHAPE);

  // grouped-query scores: workspace sizing, group out of range, short workspace, aliasing outputs
  kv_shape nolen = sh;
  nolen.seq_len = nullptr;
  const size_t need = kv_score_gqa_workspace_bytes(&nolen, 4);
  if (need != KV_WORKSPACE_HEADER + 4 * 4 * 2 * sizeof(double)) ++failures;
  if (kv_score_gqa_workspace_bytes(&nolen, 17) != 0 || kv_score_gqa_workspace_bytes(nullptr, 4) != 0) ++failures;
  float *hs = reinterpret_cast<float *>(0x100000), *sc = reinterpret_cast<float *>(0x900000);
  void *ws = reinterpret_cast<void *>(0xA00000);
  EXPECT(tri_score_gqa(&sh, dummy, nullptr, 17, (const float *)dummy, nullptr, seq, 1e4, deltas, 3, hs, sc, ws, need, nullptr), KV_EINVAL);
  EXPECT(tri_score_gqa(&sh, dummy, nullptr, 4, (const float *)dummy, nullptr, seq, 1e4, deltas, 3, hs, sc, ws, need - 8, nullptr), KV_EWORKSPACE);
  EXPECT(tri_score_gqa(&sh, dummy, nullptr, 4, (const float *)dummy, nullptr, seq, 1e4, deltas, 3, hs, hs, ws, need, nullptr), KV_EINVAL);

  // the allocation-free grouped-query form: a shape whose partial sums exceed its array, a bad group
  if (kv_score_gqa_noalloc_max_bytes() < (size_t{1} << 20)) ++failures;
  {
    kv_shape big{36, 8, 8, 128, 32768, KV_BF16, seq};
    EXPECT(tri_score_gqa_noalloc(&big, dummy, nullptr, 16, (const float *)dummy, nullptr, seq, 1e4, deltas, 3, hs, sc, nullptr), KV_EWORKSPACE);
    EXPECT(tri_score_gqa_noalloc(&sh, dummy, nullptr, 17, (const float *)dummy, nullptr, seq, 1e4, deltas, 3, hs, sc, nullptr), KV_EINVAL);
  }

  // grouped-query scores of rotated keys: group beyond 8, head_dim beyond one piece per lane,
  // half-split rows that do not fill whole lanes, unknown pool layout
  EXPECT(tri_score_gqa_rotated(&sh, dummy, nullptr, 0, 9, (const float *)dummy, nullptr, seq, 1e4, deltas, 3, hs, sc, ws, need, nullptr), KV_EINVAL);
  kv_shape sh256 = sh;
  sh256.head_dim = 256;
  EXPECT(tri_score_gqa_rotated(&sh256, dummy, nullptr, 0, 4, (const float *)dummy, nullptr, seq, 1e4, deltas, 3, hs, sc, ws, 1 << 20, nullptr), KV_ESHAPE);
  kv_shape sh96 = sh;
  sh96.head_dim = 96;
  EXPECT(tri_score_gqa_rotated(&sh96, dummy, nullptr, 1, 4, (const float *)dummy, nullptr, seq, 1e4, deltas, 3, hs, sc, ws, need, nullptr), KV_ESHAPE);
  kv_paged pg3{seq, 256, 16, 8, 3};
  EXPECT(tri_score_gqa_rotated(&sh, dummy, &pg3, 0, 4, (const float *)dummy, nullptr, seq, 1e4, deltas, 3, hs, sc, ws, need, nullptr), KV_EINVAL);

  // workspace queries and rejections: a missing, misaligned or short workspace
  if (kv_score_workspace_bytes(&nolen, 3) != KV_WORKSPACE_HEADER || kv_score_workspace_bytes(&nolen, 0) != 0) ++failures;
  const size_t need_sel = kv_select_workspace_bytes(&nolen, 1024);
  if (need_sel < KV_WORKSPACE_HEADER || kv_select_workspace_bytes(&nolen, 0) != 0) ++failures;
  EXPECT(tri_score(&sh, dummy, nullptr, (const float *)dummy, nullptr, seq, 1e4, deltas, 3, (float *)dummy, nullptr, 1 << 20, nullptr), KV_EWORKSPACE);
  EXPECT(tri_score(&sh, dummy, nullptr, (const float *)dummy, nullptr, seq, 1e4, deltas, 3, (float *)dummy, (void *)0x7000004, 1 << 20, nullptr), KV_EWORKSPACE);
  EXPECT(tri_score(&sh, dummy, nullptr, (const float *)dummy, nullptr, seq, 1e4, deltas, 3, (float *)dummy, wsp, KV_WORKSPACE_HEADER - 1, nullptr), KV_EWORKSPACE);
  {
    int32_t *k = reinterpret_cast<int32_t *>(0x3000), *n = reinterpret_cast<int32_t *>(0x4000);
    EXPECT(kv_select_topk(&sh, &pol, (const float *)dummy, k, 1024, n, wsp, need_sel - 1, nullptr), KV_EWORKSPACE);
    EXPECT(kv_select_random(&sh, &pol, nullptr, 1, 0, 0, k, 1024, n, nullptr, need_sel, nullptr), KV_EWORKSPACE);
    EXPECT(kv_select_random(&sh, &pol, nullptr, 1, 0, -1, k, 1024, n, wsp, need_sel, nullptr), KV_EINVAL);
    EXPECT(kv_select_random(&sh, &pol, nullptr, 1, 0, 65536, k, 1024, n, wsp, need_sel, nullptr), KV_EINVAL);
    EXPECT(kv_select_random_shared(&sh, &pol, nullptr, 1, 0, k, 1024, n, (void *)0x7000004, need_sel, nullptr), KV_EWORKSPACE);
  }

  // selectors: b_cap below the budget, t_cap past every selector (2^26) or past the union's
  // limit (2^18), budget < 1, union without head scores
  int32_t *kept = reinterpret_cast<int32_t *>(0x3000), *nk = reinterpret_cast<int32_t *>(0x4000);
  EXPECT(kv_select_topk(&sh, &pol, (const float *)dummy, kept, 1000, nk, wsp, 1 << 20, nullptr), KV_ESHAPE);
  kv_shape big = sh;
  big.t_cap = (1 << 26) + 1;
  EXPECT(kv_select_topk(&big, &pol, (const float *)dummy, kept, 1024, nk, wsp, 1 << 20, nullptr), KV_ESHAPE);
  EXPECT(kv_select_random(&big, &pol, nullptr, 1, 0, 0, kept, 1024, nk, wsp, 1 << 20, nullptr), KV_ESHAPE);
  EXPECT(kv_select_random_shared(&big, &pol, nullptr, 1, 0, kept, 1024, nk, wsp, 1 << 20, nullptr), KV_ESHAPE);
  big.t_cap = (1 << 18) + 1;
  EXPECT(kv_select_union(&big, &pol, 4, 0, (const float *)dummy, (const float *)dummy, kept, 1024, nk, nullptr), KV_ESHAPE);
  kv_policy zero = pol;
  zero.budget = 0;
  EXPECT(kv_select_recent(&sh, &zero, kept, 1024, nk, nullptr), KV_EINVAL);
  EXPECT(kv_select_union(&sh, &pol, 4, 0, nullptr, (const float *)dummy, kept, 1024, nk, nullptr), KV_EINVAL);
  EXPECT(kv_audit_kept(&sh, &pol, kept, 1024, nk, nullptr, nullptr), KV_EINVAL);

  // compaction: overlapping input and output, overlapping in-place K and V
  void *a = reinterpret_cast<void *>(0x1000000);
  EXPECT(kv_compact(&sh, a, (void *)0x2000000, nullptr, kept, 1024, nk, a, (void *)0x3000000, nullptr, 1024, nullptr), KV_EINVAL);
  EXPECT(kv_compact_inplace(&sh, a, (void *)0x1000010, nullptr, kept, 1024, nk, nullptr), KV_EINVAL);

  // measurement aid: NULL or misaligned pointers, a size that is not a whole number of 128 KB
  uint32_t *o = reinterpret_cast<uint32_t *>(0x5000);
  EXPECT(kv_stream_ceiling(nullptr, 131072, o, 1, nullptr), KV_EINVAL);
  EXPECT(kv_stream_ceiling(a, 131072, nullptr, 0, nullptr), KV_EINVAL);
  EXPECT(kv_stream_ceiling((void *)0x1000008, 131072, o, 1, nullptr), KV_EINVAL);
  EXPECT(kv_stream_ceiling(a, 131072, (uint32_t *)0x5002, 1, nullptr), KV_EINVAL);
  EXPECT(kv_stream_ceiling(a, 0, o, 1, nullptr), KV_EINVAL);
  EXPECT(kv_stream_ceiling(a, 131072 + 4096, o, 1, nullptr), KV_EINVAL);
  EXPECT(kv_stream_ceiling(a, static_cast<size_t>(1) << 48, o, 1, nullptr), KV_ESHAPE);

  if (failures) std::fprintf(stderr, "%d failures\n", failures);
  else std::printf("host checks ok\n");
  return failures ? 1 : 0;
}

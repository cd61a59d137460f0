// C ABI of the KV-eviction hot path: argument validation, the fp64 fold of the
// offset average, and kernel launches. See include/kvevict.h for the contract.
#include <cmath>
#include <cstdint>
#include <initializer_list>
#include <mutex>

#include "kvevict.h"
#include "kv_internal.hpp"

#define KV_EXPORT extern "C" __attribute__((visibility("default")))

// A build with -DKV_DEVICE_CHECKS=1 (libkvevict_debug.so) launches the precondition kernel of
// checks.hip before each call's own kernels; the release build does not.
#ifndef KV_DEVICE_CHECKS
#define KV_DEVICE_CHECKS 0
#endif

namespace kvevict {
namespace {

constexpr double kTwoPi = 6.283185307179586476925286766559;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// 4-byte element arrays (int32 / fp32) are read and written as whole words; NULL passes (optional
// arguments are checked for presence separately)
bool words(std::initializer_list<const void *> ps) {
  for (const void *p : ps)
    if (reinterpret_cast<uintptr_t>(p) & 3u) return false;
  return true;
}

// Selectors never touch K/V rows, so they ignore head_dim and dtype (rows == false).
// need_len == false: only the sizes are checked (workspace queries take no device arrays).
kv_status check_shape(const kv_shape *sh, bool rows, bool need_len = true) {
  if (!sh || (need_len && !sh->seq_len)) return KV_EINVAL;
  if (sh->n_layers < 1 || sh->n_layers >= 65536 || sh->n_seq < 1 || sh->n_kv_heads < 1 ||
      sh->n_kv_heads >= 65536 || sh->t_cap < 1)
    return KV_EINVAL;
  const long long heads = static_cast<long long>(sh->n_layers) * sh->n_seq * sh->n_kv_heads;
  if (heads > (1ll << 31) - 1) return KV_ESHAPE;
  if (!rows) return KV_OK;
  if (sh->dtype != KV_F32 && sh->dtype != KV_BF16) return KV_EDTYPE;
  const int d = sh->head_dim;
  if (d < 2 || d > 2 * kMaxBands || (d % 2)) return KV_ESHAPE;
  if (sh->dtype == KV_BF16 && d % 8) return KV_ESHAPE;
  if (sh->dtype == KV_F32 && d % 4) return KV_ESHAPE;
  return KV_OK;
}

kv_status check_policy(const kv_policy *po, int b_cap) {
  if (!po || !po->prompt_len) return KV_EINVAL;
  if (po->budget < 1 || po->recent < 0 || po->prompt_cap < 0) return KV_EINVAL;
  if (b_cap < po->budget || b_cap < po->prompt_cap) return KV_ESHAPE;
  return KV_OK;
}

kv_status hip_status(hipError_t e) { return e == hipSuccess ? KV_OK : KV_EHIP; }

// Every workspace starts with the header (status word + reserved bytes); kernel scratch follows.
kv_status check_workspace(const void *ws, size_t bytes, size_t need) {
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 7u) || bytes < need) return KV_EWORKSPACE;
  return KV_OK;
}

// Debug build: verify the device-side preconditions (lengths, prompt lengths, position order) and
// OR the KV_DEV_* bits of what fails into the workspace status word. Release build: nothing.
kv_status device_checks(const kv_shape *sh, const kv_policy *po, const int32_t *pos, void *ws, hipStream_t st) {
  if (!KV_DEVICE_CHECKS) return KV_OK;
  CheckParams c{};
  c.seq_len = sh->seq_len;
  c.prompt_len = po ? po->prompt_len : nullptr;
  c.prompt_cap = po ? po->prompt_cap : 0;
  c.pos = pos;
  c.L = sh->n_layers;
  c.S = sh->n_seq;
  c.H = sh->n_kv_heads;
  c.t_cap = sh->t_cap;
  c.status = static_cast<uint32_t *>(ws);
  return hip_status(launch_device_checks(c, st));
}

// Band frequencies omega_f = theta^(-2f/d) (as revolutions per position, omega_f / 2pi) and the
// fold coefficient A_f = (1/|D|) sum_delta exp(i omega_f delta), both in fp64 with the phase
// reduced to [-1/2, 1/2] revolutions before sin/cos.
void fold_coefficients(int d, double rope_theta, const int32_t *deltas, int n_delta, float2 *A, double *rev_out) {
  for (int f = 0; f < d / 2; ++f) {
    const double omega = std::pow(rope_theta, -2.0 * f / d);
    const double rev = omega / kTwoPi;
    double re = 0.0, im = 0.0;
    for (int i = 0; i < n_delta; ++i) {
      const double x = rev * static_cast<double>(deltas[i]);
      const double r = x - std::nearbyint(x);
      re += std::cos(kTwoPi * r);
      im += std::sin(kTwoPi * r);
    }
    A[f] = make_float2(static_cast<float>(re / n_delta), static_cast<float>(im / n_delta));
    rev_out[f] = rev;
  }
}

int elem_bytes(const kv_shape *sh) { return sh->dtype == KV_BF16 ? 2 : 4; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

}  // namespace
}  // namespace kvevict

using namespace kvevict;

KV_EXPORT int32_t kv_version(void) { return (2 << 16) | 1; }

KV_EXPORT int32_t kv_device_checks(void) { return KV_DEVICE_CHECKS ? 1 : 0; }

KV_EXPORT const char *kv_status_string(int32_t status) {
  switch (status) {
    case KV_OK: return "ok";
    case KV_EINVAL: return "invalid argument (null pointer, non-positive size, bad policy or aliasing)";
    case KV_EDTYPE: return "unknown element type";
    case KV_ESHAPE: return "shape or capacity outside what the kernels support";
    case KV_EWORKSPACE: return "workspace missing, misaligned or smaller than its *_workspace_bytes query";
    case KV_EHIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

KV_EXPORT size_t kv_score_workspace_bytes(const kv_shape *shape, int32_t n_delta) {
  if (check_shape(shape, true, false) != KV_OK || n_delta < 1 || n_delta > kMaxDeltas) return 0;
  return kWorkspaceHeader;   // the score stream needs no scratch of its own
}

KV_EXPORT kv_status tri_score(const kv_shape *shape, const void *K, const int32_t *pos, const float *qbar,
                              const float *qabs, const int32_t *t_cur, double rope_theta, const int32_t *deltas,
                              int32_t n_delta, float *scores, void *workspace, size_t workspace_bytes,
                              void *stream) {
  kv_status st = check_shape(shape, true);
  if (st != KV_OK) return st;
  if (!K || !qbar || !t_cur || !deltas || !scores) return KV_EINVAL;
  if (!(rope_theta > 0.0) || !std::isfinite(rope_theta)) return KV_EINVAL;
  if (n_delta < 1 || n_delta > kMaxDeltas) return KV_EINVAL;
  if (!aligned16(K) || (reinterpret_cast<uintptr_t>(qbar) & 7u)) return KV_EINVAL;
  if (!words({pos, qabs, t_cur, scores, shape->seq_len})) return KV_EINVAL;
  if ((st = check_workspace(workspace, workspace_bytes, kWorkspaceHeader)) != KV_OK) return st;

  ScoreParams p{};
  p.K = K;
  p.pos = pos;
  p.qbar = qbar;
  p.qabs = qabs;
  p.t_cur = t_cur;
  p.seq_len = shape->seq_len;
  p.scores = scores;
  p.L = shape->n_layers;
  p.S = shape->n_seq;
  p.H = shape->n_kv_heads;
  p.d = shape->head_dim;
  p.F = shape->head_dim / 2;
  p.t_cap = shape->t_cap;
  p.chunks_per_head = (shape->t_cap + kScoreChunk - 1) / kScoreChunk;

  fold_coefficients(p.d, rope_theta, deltas, n_delta, p.A, p.rev);
  // one head's rows are addressed with 32-bit buffer offsets
  if (static_cast<long long>(p.t_cap) * p.d * elem_bytes(shape) + (64ll << 9) >= (1ll << 31)) return KV_ESHAPE;
  const int bpl = shape->dtype == KV_BF16 ? 4 : 2;  // bands per 16-byte lane piece
  const int pieces = (p.F + bpl - 1) / bpl;
  int lpk = 1;
  while (lpk < pieces) lpk <<= 1;
  if (lpk > 64) return KV_ESHAPE;
  const long long threads = static_cast<long long>(p.L) * p.S * p.H * p.chunks_per_head * kScoreThreads;
  if (threads >= (1ll << 32)) return KV_ESHAPE;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = device_checks(shape, nullptr, pos, workspace, hs)) != KV_OK) return st;
  return hip_status(launch_score(p, shape->dtype == KV_BF16, lpk, hs));
}

KV_EXPORT kv_status tri_score_rotated(const kv_shape *shape, const void *K, const kv_paged *paged,
                                      int32_t rope_style, const float *qbar, const float *qabs,
                                      const int32_t *t_cur, double rope_theta, const int32_t *deltas,
                                      int32_t n_delta, float *scores, void *stream) {
  kv_status st = check_shape(shape, true);
  if (st != KV_OK) return st;
  if (!K || !qbar || !t_cur || !deltas || !scores) return KV_EINVAL;
  if (!(rope_theta > 0.0) || !std::isfinite(rope_theta)) return KV_EINVAL;
  if (n_delta < 1 || n_delta > kMaxDeltas) return KV_EINVAL;
  if (rope_style != KV_ROPE_INTERLEAVED && rope_style != KV_ROPE_HALF) return KV_EINVAL;
  if (!aligned16(K) || (reinterpret_cast<uintptr_t>(qbar) & 3u)) return KV_EINVAL;
  if (!words({qabs, t_cur, scores, shape->seq_len, paged ? paged->block_table : nullptr})) return KV_EINVAL;

  RotScoreParams p{};
  p.K = K;
  p.qbar = qbar;
  p.qabs = qabs;
  p.t_cur = t_cur;
  p.seq_len = shape->seq_len;
  p.scores = scores;
  p.L = shape->n_layers;
  p.S = shape->n_seq;
  p.H = shape->n_kv_heads;
  p.d = shape->head_dim;
  p.F = shape->head_dim / 2;
  p.t_cap = shape->t_cap;
  p.half = rope_style == KV_ROPE_HALF;
  p.chunks_per_head = (shape->t_cap + kScoreChunk - 1) / kScoreChunk;
  if (paged) {
    if (paged->head_major != 0 && paged->head_major != 1) return KV_EINVAL;
    if (!paged->block_table || paged->blocks_per_seq < 1 || paged->n_blocks < 1 || paged->block_size < 1 ||
        (paged->block_size & (paged->block_size - 1)))
      return KV_EINVAL;
    if (static_cast<long long>(paged->blocks_per_seq) * paged->block_size < shape->t_cap) return KV_ESHAPE;
    p.block_table = paged->block_table;
    p.blocks_per_seq = paged->blocks_per_seq;
    p.n_blocks = paged->n_blocks;
    p.head_major = paged->head_major;
    int shift = 0;
    while ((1 << shift) < paged->block_size) ++shift;
    p.block_shift = shift;
  }
  fold_coefficients(p.d, rope_theta, deltas, n_delta, p.A, p.rev);
  const int pieces = p.d * elem_bytes(shape) / 16;  // 16-byte lane pieces per row
  int lpk = 1;
  while (lpk < pieces) lpk <<= 1;
  if (lpk > 64) return KV_ESHAPE;
  if (p.half && (lpk != pieces || lpk < 2)) return KV_ESHAPE;  // the two halves must fill whole lanes
  const long long threads = static_cast<long long>(p.L) * p.S * p.H * p.chunks_per_head * kScoreThreads;
  if (threads >= (1ll << 32)) return KV_ESHAPE;
  return hip_status(launch_score_rotated(p, shape->dtype == KV_BF16, lpk, static_cast<hipStream_t>(stream)));
}

namespace kvevict {
namespace {
// Partial sums of tri_score_gqa: per (l, s, h, score chunk, g), the fp64 sums of s and s^2.
size_t gqa_workspace(const kv_shape *sh, int group) {
  const size_t heads = static_cast<size_t>(sh->n_layers) * sh->n_seq * sh->n_kv_heads;
  const size_t chunks = (static_cast<size_t>(sh->t_cap) + kGqaChunk - 1) / kGqaChunk;
  return kWorkspaceHeader + heads * chunks * static_cast<size_t>(group) * 2 * sizeof(double);
}
}  // namespace
}  // namespace kvevict

KV_EXPORT size_t kv_score_gqa_workspace_bytes(const kv_shape *shape, int32_t group) {
  if (check_shape(shape, true, false) != KV_OK || group < 1 || group > kGqaMaxGroup) return 0;
  return gqa_workspace(shape, group);
}

KV_EXPORT kv_status tri_score_gqa(const kv_shape *shape, const void *K, const int32_t *pos, int32_t group,
                                  const float *qbar, const float *qabs, const int32_t *t_cur, double rope_theta,
                                  const int32_t *deltas, int32_t n_delta, float *head_scores, float *scores,
                                  void *workspace, size_t workspace_bytes, void *stream) {
  kv_status st = check_shape(shape, true);
  if (st != KV_OK) return st;
  if (!K || !qbar || !t_cur || !deltas || !scores || !head_scores) return KV_EINVAL;
  if (group < 1 || group > kGqaMaxGroup) return KV_EINVAL;
  if (!(rope_theta > 0.0) || !std::isfinite(rope_theta)) return KV_EINVAL;
  if (n_delta < 1 || n_delta > kMaxDeltas) return KV_EINVAL;
  if (!aligned16(K) || (reinterpret_cast<uintptr_t>(qbar) & 7u)) return KV_EINVAL;
  if (!words({pos, qabs, t_cur, head_scores, scores, shape->seq_len})) return KV_EINVAL;
  if ((st = check_workspace(workspace, workspace_bytes, gqa_workspace(shape, group))) != KV_OK) return st;
  // one head's per-query-head scores are stored through a 32-bit buffer offset
  if (static_cast<long long>(group) * shape->t_cap * 4 >= (1ll << 31)) return KV_ESHAPE;
  const size_t heads = static_cast<size_t>(shape->n_layers) * shape->n_seq * shape->n_kv_heads;
  const size_t score_bytes = heads * shape->t_cap * sizeof(float);
  if (overlaps(head_scores, score_bytes * group, scores, score_bytes) ||
      overlaps(workspace, workspace_bytes, scores, score_bytes) ||
      overlaps(workspace, workspace_bytes, head_scores, score_bytes * group))
    return KV_EINVAL;

  GqaParams p{};
  p.K = K;
  p.pos = pos;
  p.qbar = qbar;
  p.qabs = qabs;
  p.t_cur = t_cur;
  p.seq_len = shape->seq_len;
  p.raw = head_scores;
  p.partials = reinterpret_cast<double *>(static_cast<char *>(workspace) + kWorkspaceHeader);
  p.scores = scores;
  p.L = shape->n_layers;
  p.S = shape->n_seq;
  p.H = shape->n_kv_heads;
  p.d = shape->head_dim;
  p.F = shape->head_dim / 2;
  p.t_cap = shape->t_cap;
  p.G = group;
  p.chunks_per_head = (shape->t_cap + kGqaChunk - 1) / kGqaChunk;
  fold_coefficients(p.d, rope_theta, deltas, n_delta, p.A, p.rev);
  for (int f = 0; f < p.F; ++f) {  // exp(-i omega_f kGqaTile), reduced in revolutions first
    const double x = -p.rev[f] * kGqaTile;
    const double r = x - std::nearbyint(x);
    p.W[f] = make_float2(static_cast<float>(std::cos(kTwoPi * r)), static_cast<float>(std::sin(kTwoPi * r)));
  }
  const int pieces = p.d * elem_bytes(shape) / 16;   // 16-byte pieces per row, four lanes share a row
  int ppq = 1;
  while (4 * ppq < pieces) ppq <<= 1;
  if (ppq > 8) return KV_ESHAPE;
  const long long threads = static_cast<long long>(p.L) * p.S * p.H * p.chunks_per_head * kScoreThreads;
  if (threads >= (1ll << 32)) return KV_ESHAPE;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = device_checks(shape, nullptr, pos, workspace, hs)) != KV_OK) return st;
  return hip_status(launch_score_gqa(p, shape->dtype == KV_BF16, ppq, hs));
}

// ---- tri_score_gqa without a caller workspace (for callers that cannot allocate) ----
//
// The partial sums live in a file-scope device array instead. In host code `gqa_scratch` names a
// host-side stand-in, not device memory: its device address is taken once per device with
// hipGetSymbolAddress (with that device current) and only that address reaches the kernels.
namespace kvevict {
namespace {
constexpr size_t kStaticScratchBytes = size_t{8} << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char gqa_scratch[kStaticScratchBytes];
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];   // device address of gqa_scratch on each device, once taken

// The current device's copy of gqa_scratch, or nullptr when its address cannot be taken.
void *device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(gqa_scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace
}  // namespace kvevict

KV_EXPORT size_t kv_score_gqa_noalloc_max_bytes(void) { return kStaticScratchBytes; }

KV_EXPORT kv_status tri_score_gqa_noalloc(const kv_shape *shape, const void *K, const int32_t *pos, int32_t group,
                                          const float *qbar, const float *qabs, const int32_t *t_cur,
                                          double rope_theta, const int32_t *deltas, int32_t n_delta,
                                          float *head_scores, float *scores, void *stream) {
  kv_status st = check_shape(shape, true);
  if (st != KV_OK) return st;
  if (group < 1 || group > kGqaMaxGroup) return KV_EINVAL;
  if (gqa_workspace(shape, group) > kStaticScratchBytes) return KV_EWORKSPACE;   // beyond the static array
  void *ws = device_scratch();
  if (!ws) return KV_EHIP;
  return tri_score_gqa(shape, K, pos, group, qbar, qabs, t_cur, rope_theta, deltas, n_delta, head_scores, scores, ws,
                       kStaticScratchBytes, stream);
}

// max_slots: the largest t_cap the selector kernel behind the entry point takes.
KV_EXPORT kv_status tri_score_gqa_rotated(const kv_shape *shape, const void *K, const kv_paged *paged,
                                          int32_t rope_style, int32_t group, const float *qbar, const float *qabs,
                                          const int32_t *t_cur, double rope_theta, const int32_t *deltas,
                                          int32_t n_delta, float *head_scores, float *scores, void *workspace,
                                          size_t workspace_bytes, void *stream) {
  kv_status st = check_shape(shape, true);
  if (st != KV_OK) return st;
  if (!K || !qbar || !t_cur || !deltas || !scores || !head_scores) return KV_EINVAL;
  if (group < 1 || group > kGqaRotatedMaxGroup) return KV_EINVAL;
  if (!(rope_theta > 0.0) || !std::isfinite(rope_theta)) return KV_EINVAL;
  if (n_delta < 1 || n_delta > kMaxDeltas) return KV_EINVAL;
  if (rope_style != KV_ROPE_INTERLEAVED && rope_style != KV_ROPE_HALF) return KV_EINVAL;
  if (!aligned16(K) || (reinterpret_cast<uintptr_t>(qbar) & 3u)) return KV_EINVAL;
  if (!words({qabs, t_cur, head_scores, scores, shape->seq_len, paged ? paged->block_table : nullptr}))
    return KV_EINVAL;
  if ((st = check_workspace(workspace, workspace_bytes, gqa_workspace(shape, group))) != KV_OK) return st;
  const size_t heads = static_cast<size_t>(shape->n_layers) * shape->n_seq * shape->n_kv_heads;
  const size_t score_bytes = heads * shape->t_cap * sizeof(float);
  if (overlaps(head_scores, score_bytes * group, scores, score_bytes) ||
      overlaps(workspace, workspace_bytes, scores, score_bytes) ||
      overlaps(workspace, workspace_bytes, head_scores, score_bytes * group))
    return KV_EINVAL;

  GqaParams p{};
  p.K = K;
  p.qbar = qbar;
  p.qabs = qabs;
  p.t_cur = t_cur;
  p.seq_len = shape->seq_len;
  p.raw = head_scores;
  p.partials = reinterpret_cast<double *>(static_cast<char *>(workspace) + kWorkspaceHeader);
  p.scores = scores;
  p.L = shape->n_layers;
  p.S = shape->n_seq;
  p.H = shape->n_kv_heads;
  p.d = shape->head_dim;
  p.F = shape->head_dim / 2;
  p.t_cap = shape->t_cap;
  p.G = group;
  p.chunks_per_head = (shape->t_cap + kGqaChunk - 1) / kGqaChunk;
  p.half = rope_style == KV_ROPE_HALF;
  int layout = 0;
  if (paged) {
    if (paged->head_major != 0 && paged->head_major != 1) return KV_EINVAL;
    if (!paged->block_table || paged->blocks_per_seq < 1 || paged->n_blocks < 1 || paged->block_size < 1 ||
        (paged->block_size & (paged->block_size - 1)))
      return KV_EINVAL;
    if (static_cast<long long>(paged->blocks_per_seq) * paged->block_size < shape->t_cap) return KV_ESHAPE;
    p.block_table = paged->block_table;
    p.blocks_per_seq = paged->blocks_per_seq;
    p.n_blocks = paged->n_blocks;
    int shift = 0;
    while ((1 << shift) < paged->block_size) ++shift;
    p.block_shift = shift;
    layout = paged->head_major ? 2 : 1;
  }
  fold_coefficients(p.d, rope_theta, deltas, n_delta, p.A, p.rev);
  const int pieces = p.d * elem_bytes(shape) / 16;  // 16-byte lane pieces per row
  int lpk = 1;
  while (lpk < pieces) lpk <<= 1;
  if (lpk > 16) return KV_ESHAPE;                     // one piece per lane, at most 16 lanes per key
  if (p.half && (lpk != pieces || lpk < 2)) return KV_ESHAPE;
  // one head's per-query-head scores are addressed with 32-bit offsets
  if (static_cast<long long>(group) * shape->t_cap * 4 >= (1ll << 31)) return KV_ESHAPE;
  const long long threads = static_cast<long long>(p.L) * p.S * p.H * p.chunks_per_head * kScoreThreads;
  if (threads >= (1ll << 32)) return KV_ESHAPE;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = device_checks(shape, nullptr, nullptr, workspace, hs)) != KV_OK) return st;
  return hip_status(launch_score_gqa_rotated(p, shape->dtype == KV_BF16, layout, lpk, hs));
}

static kv_status select_common(const kv_shape *shape, const kv_policy *policy, int32_t *kept, int32_t b_cap,
                               int32_t *n_kept, SelectParams &p, int max_slots = kSelectMaxSlotsStream) {
  kv_status st = check_shape(shape, false);
  if (st != KV_OK) return st;
  if ((st = check_policy(policy, b_cap)) != KV_OK) return st;
  if (!kept || !n_kept) return KV_EINVAL;
  if (!words({kept, n_kept, shape->seq_len, policy->prompt_len})) return KV_EINVAL;
  if (shape->t_cap > max_slots) return KV_ESHAPE;
  p.seq_len = shape->seq_len;
  p.prompt_len = policy->prompt_len;
  p.kept = kept;
  p.n_kept = n_kept;
  p.L = shape->n_layers;
  p.S = shape->n_seq;
  p.H = shape->n_kv_heads;
  p.t_cap = shape->t_cap;
  p.b_cap = b_cap;
  p.budget = policy->budget;
  p.recent = policy->recent;
  p.prompt_cap = policy->prompt_cap;
  return KV_OK;
}

KV_EXPORT size_t kv_select_workspace_bytes(const kv_shape *shape, int32_t b_cap) {
  if (check_shape(shape, false, false) != KV_OK || b_cap < 1 || shape->t_cap > kSelectMaxSlotsStream) return 0;
  return kWorkspaceHeader + select_scratch_bytes(shape->n_layers, shape->n_seq, shape->n_kv_heads, shape->t_cap);
}

// The selectors' workspace: validated against the query, scratch after the header.
static kv_status select_workspace(const kv_shape *shape, void *ws, size_t bytes, SelectParams &p) {
  const size_t scratch = select_scratch_bytes(shape->n_layers, shape->n_seq, shape->n_kv_heads, shape->t_cap);
  kv_status st = check_workspace(ws, bytes, kWorkspaceHeader + scratch);
  if (st != KV_OK) return st;
  p.scratch = scratch ? static_cast<char *>(ws) + kWorkspaceHeader : nullptr;
  return KV_OK;
}

KV_EXPORT kv_status kv_select_topk(const kv_shape *shape, const kv_policy *policy, const float *scores,
                                   int32_t *kept, int32_t b_cap, int32_t *n_kept, void *workspace,
                                   size_t workspace_bytes, void *stream) {
  SelectParams p{};
  kv_status st = select_common(shape, policy, kept, b_cap, n_kept, p);
  if (st != KV_OK) return st;
  if (!scores || !words({scores})) return KV_EINVAL;
  if ((st = select_workspace(shape, workspace, workspace_bytes, p)) != KV_OK) return st;
  p.scores = scores;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = device_checks(shape, policy, nullptr, workspace, hs)) != KV_OK) return st;
  return hip_status(launch_select(p, SelectKind::kTopk, hs));
}

static kv_status select_random(const kv_shape *shape, const kv_policy *policy, const int32_t *pos, uint64_t seed,
                               uint32_t event, int32_t layer_base, int32_t *kept, int32_t b_cap, int32_t *n_kept,
                               void *workspace, size_t workspace_bytes, void *stream, int shared_draw) {
  SelectParams p{};
  kv_status st = select_common(shape, policy, kept, b_cap, n_kept, p);
  if (st != KV_OK) return st;
  if (!words({pos})) return KV_EINVAL;
  // the counter packs the layer into 16 bits
  if (layer_base < 0 || static_cast<long long>(layer_base) + shape->n_layers > 65536) return KV_EINVAL;
  p.layer_base = layer_base;
  if ((st = select_workspace(shape, workspace, workspace_bytes, p)) != KV_OK) return st;
  p.pos = pos;
  p.seed_lo = static_cast<uint32_t>(seed & 0xffffffffu);
  p.seed_hi = static_cast<uint32_t>(seed >> 32);
  p.event = event;
  p.shared_draw = shared_draw;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = device_checks(shape, policy, pos, workspace, hs)) != KV_OK) return st;
  return hip_status(launch_select(p, SelectKind::kRandom, hs));
}

KV_EXPORT kv_status kv_select_random(const kv_shape *shape, const kv_policy *policy, const int32_t *pos,
                                     uint64_t seed, uint32_t event, int32_t layer_base, int32_t *kept,
                                     int32_t b_cap, int32_t *n_kept, void *workspace, size_t workspace_bytes,
                                     void *stream) {
  return select_random(shape, policy, pos, seed, event, layer_base, kept, b_cap, n_kept, workspace, workspace_bytes,
                       stream, 0);
}

KV_EXPORT kv_status kv_select_union(const kv_shape *shape, const kv_policy *policy, int32_t group,
                                    int32_t k_per_head, const float *head_scores, const float *scores,
                                    int32_t *kept, int32_t b_cap, int32_t *n_kept, void *stream) {
  SelectParams p{};
  kv_status st = select_common(shape, policy, kept, b_cap, n_kept, p, kSelectMaxSlotsUnion);
  if (st != KV_OK) return st;
  if (!head_scores || !scores || !words({head_scores, scores})) return KV_EINVAL;
  if (group < 1 || group > 64) return KV_EINVAL;
  p.scores = scores;
  p.head_scores = head_scores;
  p.G = group;
  p.k_per_head = k_per_head;
  return hip_status(launch_select(p, SelectKind::kUnion, static_cast<hipStream_t>(stream)));
}

KV_EXPORT kv_status kv_audit_kept(const kv_shape *shape, const kv_policy *policy, const int32_t *kept,
                                  int32_t b_cap, const int32_t *n_kept, int32_t *bad, void *stream) {
  SelectParams p{};
  kv_status st = select_common(shape, policy, const_cast<int32_t *>(kept), b_cap, const_cast<int32_t *>(n_kept), p);
  if (st != KV_OK) return st;
  if (!bad || !words({bad})) return KV_EINVAL;
  return hip_status(launch_audit(p, bad, static_cast<hipStream_t>(stream)));
}

KV_EXPORT kv_status kv_stream_ceiling(const void *buf, size_t bytes, uint32_t *out, int32_t with_stores, void *stream) {
  if (!buf || !out || !aligned16(buf) || !words({out})) return KV_EINVAL;
  if (bytes == 0 || bytes % kStreamCeilingChunk != 0) return KV_EINVAL;
  if (bytes / kStreamCeilingChunk >= (1ull << 31)) return KV_ESHAPE;
  return hip_status(launch_stream_ceiling(buf, bytes, out, with_stores != 0,
                                          static_cast<hipStream_t>(stream)));
}

KV_EXPORT kv_status kv_select_random_shared(const kv_shape *shape, const kv_policy *policy, const int32_t *pos,
                                          uint64_t seed, uint32_t event, int32_t *kept, int32_t b_cap,
                                          int32_t *n_kept, void *workspace, size_t workspace_bytes, void *stream) {
  return select_random(shape, policy, pos, seed, event, 0, kept, b_cap, n_kept, workspace, workspace_bytes, stream, 1);
}

KV_EXPORT kv_status kv_select_recent(const kv_shape *shape, const kv_policy *policy, int32_t *kept, int32_t b_cap,
                                     int32_t *n_kept, void *stream) {
  SelectParams p{};
  kv_status st = select_common(shape, policy, kept, b_cap, n_kept, p);
  if (st != KV_OK) return st;
  const long long blocks = static_cast<long long>(p.L) * p.S * p.H * ((b_cap + 255) / 256);
  if (blocks >= (1ll << 31)) return KV_ESHAPE;
  return hip_status(launch_select_recent(p, static_cast<hipStream_t>(stream)));
}

KV_EXPORT kv_status kv_compact_inplace(const kv_shape *shape, void *K, void *V, int32_t *pos, const int32_t *kept,
                                       int32_t b_cap, const int32_t *n_kept, void *stream) {
  kv_status st = check_shape(shape, true);
  if (st != KV_OK) return st;
  if (!K || !V || !kept || !n_kept) return KV_EINVAL;
  if (b_cap < 1) return KV_EINVAL;
  if (!aligned16(K) || !aligned16(V)) return KV_EINVAL;
  if (!words({pos, kept, n_kept, shape->seq_len})) return KV_EINVAL;
  const size_t heads = static_cast<size_t>(shape->n_layers) * shape->n_seq * shape->n_kv_heads;
  const size_t row_bytes = static_cast<size_t>(shape->head_dim) * elem_bytes(shape);
  const size_t bytes = heads * shape->t_cap * row_bytes;
  if (overlaps(K, bytes, V, bytes)) return KV_EINVAL;
  if (pos && (overlaps(pos, heads * shape->t_cap * 4, K, bytes) || overlaps(pos, heads * shape->t_cap * 4, V, bytes)))
    return KV_EINVAL;

  HoleParams p{};
  p.K = static_cast<uint4 *>(K);
  p.V = static_cast<uint4 *>(V);
  p.pos = pos;
  p.kept = kept;
  p.n_kept = n_kept;
  p.L = shape->n_layers;
  p.S = shape->n_seq;
  p.H = shape->n_kv_heads;
  p.t_cap = shape->t_cap;
  p.b_cap = b_cap;
  p.row16 = static_cast<int32_t>(row_bytes / 16);
  // movers per head are at most min(n_kept, T - n_kept) <= t_cap / 2; about 1024 of them per workgroup
  const int max_movers = (b_cap < shape->t_cap / 2 ? b_cap : shape->t_cap / 2);
  int wgs = (max_movers + 1023) / 1024;
  p.wgs_per_head = wgs < 1 ? 1 : (wgs > 32 ? 32 : wgs);
  const long long threads = static_cast<long long>(heads) * p.wgs_per_head * 256;
  if (threads >= (1ll << 32)) return KV_ESHAPE;
  return hip_status(launch_compact_holes(p, static_cast<hipStream_t>(stream)));
}

KV_EXPORT kv_status kv_compact(const kv_shape *shape, const void *K_in, const void *V_in, const int32_t *pos_in,
                               const int32_t *kept, int32_t b_cap, const int32_t *n_kept, void *K_out,
                               void *V_out, int32_t *pos_out, int32_t out_cap, void *stream) {
  kv_status st = check_shape(shape, true);
  if (st != KV_OK) return st;
  if (!K_in || !V_in || !kept || !n_kept || !K_out || !V_out) return KV_EINVAL;
  if (b_cap < 1 || out_cap < 1) return KV_EINVAL;
  if (!aligned16(K_in) || !aligned16(V_in) || !aligned16(K_out) || !aligned16(V_out)) return KV_EINVAL;
  if (!words({pos_in, kept, n_kept, pos_out, shape->seq_len})) return KV_EINVAL;
  const size_t heads = static_cast<size_t>(shape->n_layers) * shape->n_seq * shape->n_kv_heads;
  const size_t row_bytes = static_cast<size_t>(shape->head_dim) * elem_bytes(shape);
  const size_t in_bytes = heads * shape->t_cap * row_bytes, out_bytes = heads * out_cap * row_bytes;
  if (overlaps(K_in, in_bytes, K_out, out_bytes) || overlaps(V_in, in_bytes, V_out, out_bytes) ||
      overlaps(K_in, in_bytes, V_out, out_bytes) || overlaps(V_in, in_bytes, K_out, out_bytes) ||
      overlaps(K_out, out_bytes, V_out, out_bytes))
    return KV_EINVAL;
  if (pos_out && pos_in && overlaps(pos_in, heads * shape->t_cap * 4, pos_out, heads * out_cap * 4))
    return KV_EINVAL;

  CompactParams p{};
  p.K_in = static_cast<const uint4 *>(K_in);
  p.V_in = static_cast<const uint4 *>(V_in);
  p.pos_in = pos_in;
  p.kept = kept;
  p.n_kept = n_kept;
  p.K_out = static_cast<uint4 *>(K_out);
  p.V_out = static_cast<uint4 *>(V_out);
  p.pos_out = pos_out;
  p.L = shape->n_layers;
  p.S = shape->n_seq;
  p.H = shape->n_kv_heads;
  p.t_cap = shape->t_cap;
  p.b_cap = b_cap;
  p.out_cap = out_cap;
  p.row16 = static_cast<int32_t>(row_bytes / 16);
  int G = 1;
  while (G < p.row16) G <<= 1;
  const int rows_wg = compact_rows_per_wg(G);
  const int max_rows = b_cap < out_cap ? b_cap : out_cap;
  p.wgs_per_head = (max_rows + rows_wg - 1) / rows_wg;
  const long long threads = static_cast<long long>(heads) * p.wgs_per_head * compact_wgs_per_slice() * 256;
  if (threads >= (1ll << 32)) return KV_ESHAPE;
  return hip_status(launch_compact(p, static_cast<hipStream_t>(stream)));
}

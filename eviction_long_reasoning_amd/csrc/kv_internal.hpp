// Internal declarations shared by the kernels' translation units and the C ABI layer.
// Not part of the public interface (include/kvevict.h is).
#pragma once

#include "score_params.hpp"

namespace kvevict {

// Every caller workspace starts with this many bytes: the device status word, then reserved space.
constexpr size_t kWorkspaceHeader = 256;

// Device-side preconditions checked by a build with KV_DEVICE_CHECKS (the bits of kvevict.h's
// KV_DEV_* are ORed into *status).
struct CheckParams {
  const int32_t *seq_len;     // [S]
  const int32_t *prompt_len;  // [S] or nullptr (scoring calls)
  int32_t prompt_cap;
  const int32_t *pos;         // [L,S,H,t_cap] or nullptr
  int32_t L, S, H, t_cap;
  uint32_t *status;           // the workspace's first word
};
hipError_t launch_device_checks(const CheckParams &c, hipStream_t st);

// Keys stored after RoPE, dense or paged.
struct RotScoreParams {
  const void *K;               // dense [L,S,H,t_cap,d] or paged pool [L,n_blocks,block_size,H,d]
                               // (head-major: [L,n_blocks,H,block_size,d])
  const int32_t *block_table;  // [S, blocks_per_seq] or nullptr (dense)
  int32_t blocks_per_seq, block_shift, n_blocks, head_major;
  const float *qbar;           // [L,H,d] in the storage layout
  const float *qabs;           // [L,H,d/2] or nullptr
  const int32_t *t_cur;        // [S]
  const int32_t *seq_len;      // [S]
  float *scores;               // [L,S,H,t_cap]
  int32_t L, S, H, d, F, t_cap;
  int32_t chunks_per_head;
  int32_t half;                // 1: half-split pairing (x[f], x[f+d/2]); 0: interleaved
  float2 A[kMaxBands];
  double rev[kMaxBands];
};

hipError_t launch_score_rotated(const RotScoreParams &p, int dtype_bf16, int lanes_per_key, hipStream_t st);

// Grouped-query scores: G query-head centres per KV head, z-normalised per query head, max over G.
constexpr int kGqaMaxGroup = 16;
struct GqaParams {
  const void *K;            // [L,S,H,t_cap,d]
  const int32_t *pos;       // [L,S,H,t_cap] or nullptr
  const float *qbar;        // [L,H,G,d]
  const float *qabs;        // [L,H,G,d/2] or nullptr
  const int32_t *t_cur;     // [S]
  const int32_t *seq_len;   // [S]
  float *raw;               // [L,S,H,G,t_cap] per-query-head scores
  double *partials;         // [L,S,H,chunks_per_head,G,2]: per-chunk sums of s and s^2
  float *scores;            // [L,S,H,t_cap] max over g of the normalised scores
  int32_t L, S, H, d, F, t_cap, G;
  int32_t chunks_per_head;  // workgroups per (l,s,h), kGqaChunk keys each
  float2 A[kMaxBands];
  double rev[kMaxBands];
  float2 W[kMaxBands];      // exp(-i omega_f kGqaTile): the phase step from one key tile to the next
  // keys stored after RoPE (tri_score_gqa_rotated): pairing and, for a paged pool, the block table
  int32_t half;                // 1: half-split pairing (x[f], x[f+d/2]); 0: interleaved
  const int32_t *block_table;  // [S, blocks_per_seq] or nullptr (dense)
  int32_t blocks_per_seq, block_shift, n_blocks;
};

constexpr int kGqaTile = 16;                                   // keys per MFMA tile
constexpr int kGqaTilesPerWave = 16;
constexpr int kGqaChunk = (kScoreThreads / 64) * kGqaTilesPerWave * kGqaTile;

hipError_t launch_score_gqa(const GqaParams &p, int dtype_bf16, int pieces_per_lane, hipStream_t st);
constexpr int kGqaRotatedMaxGroup = 8;
// layout: 0 dense, 1 token-major paged pool, 2 head-major paged pool
hipError_t launch_score_gqa_rotated(const GqaParams &p, int dtype_bf16, int layout, int lanes_per_key,
                                    hipStream_t st);

// --------------------------------------------------------------- select ----
struct SelectParams {
  const float *scores;      // [L,S,H,t_cap] (top-k) or nullptr (random)
  const int32_t *pos;       // [L,S,H,t_cap] or nullptr (random counter positions)
  const int32_t *seq_len;   // [S]
  const int32_t *prompt_len;// [S]
  int32_t *kept;            // [L,S,H,b_cap]
  int32_t *n_kept;          // [S]
  int32_t L, S, H, t_cap, b_cap;
  int32_t budget, recent, prompt_cap;
  uint32_t seed_lo, seed_hi, event;
  int32_t shared_draw;      // random: every (layer, head) draws as layer 0 / head 0
  int32_t layer_base;       // random: layer l of the call draws as layer layer_base + l
  const float *head_scores; // union: [L,S,H,G,t_cap] per-query-head scores (scores = combined)
  int32_t G, k_per_head;    // union: query heads per KV head; per-head top-k (<= 0: ceil(n_sel / G))
  void *scratch;            // caller workspace past its header (select_scratch_bytes), or nullptr
  // split listing (few heads): chunk workgroups list each chunk's keys above the cut into scratch
  int32_t split_chunks;     // chunks per head (0: no split)
  int32_t split_list_cap;   // list capacity of the ranking workgroup's tier
  uint32_t *split_count;    // [heads, split_chunks] listed keys per chunk
  uint32_t *split_list;     // [heads, split_chunks, kSplitChunk, 2] (key bits, slot) per listed key
};
constexpr int kSplitChunk = 2048;   // slots per chunk workgroup (256 threads x 8)

// Scratch bytes the top-k / random selectors need past the workspace header for L*S*H heads of
// t_cap slots.
size_t select_scratch_bytes(int L, int S, int H, int t_cap);

enum class SelectKind { kTopk, kRandom, kUnion };

constexpr int kSelectMaxSlots = 32768;          // register-resident tiers
constexpr int kSelectMaxSlotsStream = 1 << 26;    // top-k and random past the tiers: keys re-read per step
constexpr int kSelectMaxSlotsUnion = 1 << 18;     // union past the tiers: a bit per slot in LDS
hipError_t launch_select(const SelectParams &p, SelectKind kind, hipStream_t st);
hipError_t launch_select_recent(const SelectParams &p, hipStream_t st);
hipError_t launch_audit(const SelectParams &p, int32_t *bad, hipStream_t st);

// -------------------------------------------------------------- compact ----
struct CompactParams {
  const uint4 *K_in, *V_in;   // rows of row16 x 16 B
  const int32_t *pos_in;      // or nullptr
  const int32_t *kept;        // [L,S,H,b_cap]
  const int32_t *n_kept;      // [S]
  uint4 *K_out, *V_out;
  int32_t *pos_out;           // or nullptr
  int32_t L, S, H, t_cap, b_cap, out_cap;
  int32_t row16;              // 16-byte chunks per row
  int32_t wgs_per_head;
};

int compact_rows_per_wg(int group);  // output rows per compact workgroup for a lane-group size
int compact_wgs_per_slice();         // workgroups per (head, row range): 2 when K and V move apart
hipError_t launch_compact(const CompactParams &p, hipStream_t st);

// In-place hole filling: kept rows at or beyond n_kept move into evicted slots below it.
struct HoleParams {
  uint4 *K, *V;               // [L,S,H,t_cap] rows of row16 x 16 B, updated in place
  int32_t *pos;               // [L,S,H,t_cap] or nullptr
  const int32_t *kept;        // [L,S,H,b_cap], ascending
  const int32_t *n_kept;      // [S]
  int32_t L, S, H, t_cap, b_cap;
  int32_t row16;
  int32_t wgs_per_head;
};

hipError_t launch_compact_holes(const HoleParams &p, hipStream_t st);

// The score stream's access pattern alone (measurement aid): bytes a multiple of 128 KB.
constexpr size_t kStreamCeilingChunk = 131072;
hipError_t launch_stream_ceiling(const void *buf, size_t bytes, uint32_t *out, bool stores, hipStream_t st);

}  // namespace kvevict

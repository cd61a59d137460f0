// Internal declarations of the pre-RoPE score stream (tri_score): its launch parameters and
// workgroup shape. Shared by score.hip and the C ABI layer; not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvevict {

constexpr int kMaxBands = 128;      // head_dim <= 256
constexpr int kMaxDeltas = 64;

// ---------------------------------------------------------------- score ----
struct ScoreParams {
  const void *K;            // [L,S,H,t_cap,d]
  const int32_t *pos;       // [L,S,H,t_cap] or nullptr
  const float *qbar;        // [L,H,d]
  const float *qabs;        // [L,H,d/2] or nullptr
  const int32_t *t_cur;     // [S]
  const int32_t *seq_len;   // [S]
  float *scores;            // [L,S,H,t_cap]
  int32_t L, S, H, d, F, t_cap;
  int32_t chunks_per_head;  // workgroups per (l,s,h)
  float2 A[kMaxBands];      // fold coefficient per band: mean over D of exp(i omega_f delta)
  double rev[kMaxBands];    // omega_f / (2 pi): revolutions per position, fp64
};

// Keys handled by one score workgroup (all lane layouts): 4 waves x 2 batches x 64 keys.
#ifndef KV_SCORE_BATCHES_PER_WAVE
#define KV_SCORE_BATCHES_PER_WAVE 2
#endif
constexpr int kScoreThreads = 256;
constexpr int kScoreBatchesPerWave = KV_SCORE_BATCHES_PER_WAVE;
constexpr int kScoreChunk = (kScoreThreads / 64) * kScoreBatchesPerWave * 64;

hipError_t launch_score(const ScoreParams &p, int dtype_bf16, int lanes_per_key, hipStream_t st);

}  // namespace kvevict


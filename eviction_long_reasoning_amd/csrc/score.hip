// Streaming key-score kernel for gfx950.
//
// What is computed (one value per cached key): the trigonometric-series term
// S_trig of "TriAttention: Efficient Long Reasoning with Trigonometric KV
// Compression" (structured summary, section 3.4, "The Trigonometric Series
// Term"), with the query replaced by its centre q_bar and averaged over the
// future offsets D ("Handling Multiple Future Positions"):
//
//   S_j = sum_f Re( u_f * conj(k_{j,f}) * exp(i omega_f (t - p_j)) ),
//   u_f = q_bar_f * A_f,   A_f = (1/|D|) sum_{delta in D} exp(i omega_f delta)
//
// The offset average enters only through A_f (angle addition, the a_f/b_f
// expansion in the same section), so every key is read exactly once.
//
// Mapping onto CDNA4:
//  * A key row is split into 16-byte pieces, one per lane (4 bands of bf16
//    or 2 bands of fp32): LPK lanes per key, KPS = 64/LPK keys per wave
//    instruction, so each wave load covers KPS consecutive rows -- a fully
//    coalesced 1 KB (bf16, d=128) global_load_dwordx4.
//  * A wave processes 64 consecutive keys as one batch of LPK steps, with all
//    the batch's loads issued before the arithmetic (up to 16 x 16 B in flight
//    per lane).
//  * The phase exp(i omega_f m) is not evaluated per key. For contiguous
//    positions each lane rotates its u_f * exp(i omega_f m) by a fixed step
//    exp(-i omega_f KPS) from one key to its next; the value is derived
//    exactly (fp64 reduction of omega_f m / 2pi to [-1/2, 1/2] revolutions,
//    then the hardware sine and cosine) once per wave, so the fp32 recurrence runs at most
//    kScoreBatchesPerWave * LPK steps. With explicit (gappy) positions the
//    phase is derived the same way for every key.
//  * The LPK per-lane partial sums of a batch are combined by a shuffle
//    reduce-scatter (LPK-1 exchanges per lane for LPK keys), after which each
//    lane holds one finished score: 64 consecutive scores leave in one
//    coalesced 256-byte store.
#include "score_params.hpp"

#include <type_traits>

#ifndef KV_SCORE_PIPELINE
#define KV_SCORE_PIPELINE 1
#endif

namespace kvevict {
namespace {

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

// exp(i 2 pi rev m): the phase is reduced in fp64 to r in [-1/2, 1/2] revolutions, then the
// hardware sine and cosine (v_sin_f32 / v_cos_f32 take revolutions) give fp32 values within
// 1.3e-7 of the exact ones over a whole revolution (measured against fp64 on 2^22 points).
__device__ __forceinline__ float2 cis_rev(double rev, double m) {
  const double x = rev * m;
  const float r = static_cast<float>(x - rint(x));
  return make_float2(__builtin_amdgcn_cosf(r), __builtin_amdgcn_sinf(r));
}

// Sum of acc[k] over the N lanes of a group (lanes differing in the low log2(N) bits);
// lane g of the group returns the sum for k = g.
// The two candidates are passed through an empty asm so that the per-lane choice stays a
// register select: left as array reads, the compiler turns the choice into a dynamically
// indexed private array (a compare/select chain over all N elements).
template <int N>
__device__ __forceinline__ float reduce_scatter(float (&acc)[N], int g) {
#pragma unroll
  for (int h = N / 2; h >= 1; h /= 2) {
    const bool upper = (g & h) != 0;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      float lo = acc[i], hi = acc[i + h];
      asm volatile("" : "+v"(lo), "+v"(hi));
      const float send = upper ? lo : hi;
      const float keep = upper ? hi : lo;
      acc[i] = keep + __shfl_xor(send, h, 64);
    }
  }
  return acc[0];
}

// 16-byte raw buffer load (global memory through a buffer resource): the per-step offset
// can ride in a scalar register, so a full batch issues its loads with no vector address math.
// Keys are read exactly once, so the loads carry the non-temporal (streaming) cache policy.
constexpr int kStreamingLoad = 2;  // cache-policy bit "nt"
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStreamingLoad);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Scores are written once and read back by the selector from HBM (far more than fits in
// cache), so the stores carry the non-temporal policy: mixed into the key stream, plain
// stores cost the read stream far more bandwidth than their own 4 bytes per key.
__device__ __forceinline__ void st_score(float *p, float x) { __builtin_nontemporal_store(x, p); }

// One lane's share of a key's score: sum over its bands of Re(v_b * conj(k_b)), plus, with
// NORM, the norm-based term cn_b * |k_b| (cn_b = (1 - R_b) E|q_b|). |k_b| uses the hardware
// square root (within 1 ulp); the library sqrtf's correctly rounded expansion made the kernel
// ALU-bound.
template <bool BF16, bool NORM>
__device__ __forceinline__ float lane_dot(const uint4 &d, const float2 *v, const float *cn) {
  constexpr int BPL = BF16 ? 4 : 2;
  const uint32_t wd[4] = {d.x, d.y, d.z, d.w};
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const float re = BF16 ? __uint_as_float(wd[i] << 16) : __uint_as_float(wd[2 * i]);
    const float im = BF16 ? __uint_as_float(wd[i] & 0xffff0000u) : __uint_as_float(wd[2 * i + 1]);
    a = fmaf(v[i].x, re, a);
    a = fmaf(v[i].y, im, a);
    if (NORM) a = fmaf(cn[i], __builtin_amdgcn_sqrtf(fmaf(re, re, im * im)), a);
  }
  return a;
}

// Norm-term weight of band b: E|q_b| - |q_bar_b| = (1 - R_b) E|q_b|, zero when E|q_b| = 0.
__device__ __forceinline__ float norm_weight_of(float qa, float2 q) {
  return qa > 0.f ? qa - sqrtf(fmaf(q.x, q.x, q.y * q.y)) : 0.f;
}
__device__ __forceinline__ float norm_weight(const float *qabs, float2 q, int b) { return norm_weight_of(qabs[b], q); }

// FULL: every lane of a key group holds bands (head_dim fills the LPK lanes exactly).
template <bool BF16, int LPK, bool POS, bool FULL, bool NORM>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(const ScoreParams p) {
  constexpr int BPL = BF16 ? 4 : 2;            // bands per lane (16 bytes)
  constexpr int KPS = 64 / LPK;                // keys per wave step
  constexpr int STEPS = LPK;                   // steps per 64-key batch
  constexpr int SUB = STEPS < 16 ? STEPS : 16; // loads in flight per lane
  constexpr int EB = BF16 ? 2 : 4;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane % LPK;
  const int kk = lane / LPK;
  const int head = blockIdx.x / p.chunks_per_head;
  const int chunk = blockIdx.x - head * p.chunks_per_head;
  const int h = head % p.H;
  const int s = (head / p.H) % p.S;
  const int l = head / (p.H * p.S);

  const int T = min(max(p.seq_len[s], 0), p.t_cap);
  const int wave_first = chunk * kScoreChunk + wave * (kScoreBatchesPerWave * 64);
  if (wave_first >= T) return;
  const double tq = static_cast<double>(p.t_cur[s]);

  const bool live = FULL || g * BPL < p.F;
  float2 u[BPL], w[BPL];
  float cn[BPL];
  double rev[BPL];
  const size_t lh = static_cast<size_t>(l) * p.H + h;
  const float2 *qrow = reinterpret_cast<const float2 *>(p.qbar + lh * p.d);
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const int b = g * BPL + i;
    if (live) {
      u[i] = cmul(qrow[b], p.A[b]);
      rev[i] = p.rev[b];
      w[i] = cis_rev(rev[i], -static_cast<double>(KPS));
      cn[i] = NORM ? norm_weight(p.qabs + lh * p.F, qrow[b], b) : 0.f;
    } else {
      u[i] = make_float2(0.f, 0.f);
      rev[i] = 0.0;
      w[i] = make_float2(1.f, 0.f);
      cn[i] = 0.f;
    }
  }

  const size_t slot0 = static_cast<size_t>(head) * p.t_cap;
  const int row_bytes = p.d * EB;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char *>(static_cast<const char *>(p.K) + slot0 * static_cast<size_t>(row_bytes)), 0,
      T * row_bytes, 0x00020000);
  const int lane_off = kk * row_bytes + (live ? g * 16 : 0);
  const int step_bytes = KPS * row_bytes;

  // Contiguous positions: the lane's keys advance by KPS slots per step and by exactly 64
  // (= LPK * KPS) per batch, so one exactly derived phase per wave seeds a recurrence of
  // kScoreBatchesPerWave * LPK steps.
  float2 v[BPL];
  if (!POS) {
    const double m0 = tq - static_cast<double>(wave_first + kk);
#pragma unroll
    for (int i = 0; i < BPL; ++i) v[i] = cmul(u[i], cis_rev(rev[i], m0));
  }
#pragma unroll 1
  for (int nb = 0; nb < kScoreBatchesPerWave; ++nb) {
    const int j0 = wave_first + nb * 64;
    if (j0 >= T) break;
    const bool full = j0 + 64 <= T;             // uniform across the wave
    const int boff = j0 * row_bytes + lane_off;
    float acc[STEPS];
#pragma unroll
    for (int st0 = 0; st0 < STEPS; st0 += SUB) {
      uint4 data[SUB];
      int32_t pj[SUB];
      if (full) {
#pragma unroll
        for (int t = 0; t < SUB; ++t) data[t] = ld16(rk, boff, (st0 + t) * step_bytes);
      } else {
        // ragged tail: slots at or past T read an in-range row; their sums feed unstored scores
#pragma unroll
        for (int t = 0; t < SUB; ++t) {
          const bool in = j0 + (st0 + t) * KPS + kk < T;
          data[t] = ld16(rk, in ? boff + (st0 + t) * step_bytes : lane_off - kk * row_bytes, 0);
        }
      }
      if (POS) {
#pragma unroll
        for (int t = 0; t < SUB; ++t) {
          const int j = min(j0 + (st0 + t) * KPS + kk, T - 1);
          pj[t] = p.pos[slot0 + j];
        }
      }
#pragma unroll
      for (int t = 0; t < SUB; ++t) {
        if (POS) {
          const double m = tq - static_cast<double>(pj[t]);
#pragma unroll
          for (int i = 0; i < BPL; ++i) v[i] = cmul(u[i], cis_rev(rev[i], m));
        }
        const float a = lane_dot<BF16, NORM>(data[t], v, cn);
        acc[st0 + t] = FULL ? a : (live ? a : 0.f);
        if (!POS) {
#pragma unroll
          for (int i = 0; i < BPL; ++i) v[i] = cmul(v[i], w[i]);
        }
      }
    }
    const float sc = reduce_scatter<STEPS>(acc, g);
    const int jj = j0 + g * KPS + kk;
    if (jj < T) st_score(p.scores + slot0 + jj, sc);
  }
}

// Contiguous positions, LPK <= 16: a software-pipelined stream. The wave issues batch 0's
// loads before its phase set-up, and the loads of batch n+1 before the arithmetic of batch n
// (two register buffers), so each wave keeps a batch of 16-byte loads in flight while it
// computes.
template <bool BF16, int LPK, bool FULL, bool NORM>
__global__ __launch_bounds__(kScoreThreads) void score_stream_kernel(const ScoreParams p) {
  static_assert(LPK <= 16, "pipelined variant holds two batches of LPK loads per lane");
  constexpr int BPL = BF16 ? 4 : 2;
  constexpr int KPS = 64 / LPK;
  constexpr int STEPS = LPK;
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int NB = kScoreBatchesPerWave;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int g = lane % LPK;
  const int kk = lane / LPK;
  const int head = blockIdx.x / p.chunks_per_head;
  const int chunk = blockIdx.x - head * p.chunks_per_head;
  const int h = head % p.H;
  const int s = (head / p.H) % p.S;
  const int l = head / (p.H * p.S);

  const int T = min(max(p.seq_len[s], 0), p.t_cap);
  const int wave_first = chunk * kScoreChunk + wave * (NB * 64);
  if (wave_first >= T) return;
  const int nbat = min(NB, (T - wave_first + 63) / 64);

  const bool live = FULL || g * BPL < p.F;
  const size_t slot0 = static_cast<size_t>(head) * p.t_cap;
  const int row_bytes = p.d * EB;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char *>(static_cast<const char *>(p.K) + slot0 * static_cast<size_t>(row_bytes)), 0,
      T * row_bytes, 0x00020000);
  const int piece = live ? g * 16 : 0;
  const int lane_off = kk * row_bytes + piece;
  const int step_bytes = KPS * row_bytes;

  // The per-lane set-up inputs (query centre, fold coefficient, frequency, norm weight) are read
  // before the key batches go out: the load counter completes in order, so waiting for an input
  // read after the keys would also wait for the keys.
  const double tq = static_cast<double>(p.t_cur[s]);
  const size_t lh = static_cast<size_t>(l) * p.H + h;
  const float2 *qrow = reinterpret_cast<const float2 *>(p.qbar + lh * p.d);
  float2 qv[BPL], av[BPL];
  double rv[BPL];
  float qa[BPL];
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const int b = g * BPL + i;
    qv[i] = av[i] = make_float2(0.f, 0.f);
    rv[i] = 0.0;
    qa[i] = 0.f;
    if (live) {
      qv[i] = qrow[b];
      av[i] = p.A[b];
      rv[i] = p.rev[b];
      if (NORM) qa[i] = p.qabs[lh * p.F + b];
    }
  }
  // The body, generated twice: for a wave whose batches all lie below T (every wave of a head but
  // its last) the loads take no branch, so the compiler can count each wait to the batch it needs.
  auto body = [&](auto all_below_T) {
    constexpr bool ALL = decltype(all_below_T)::value;
    auto issue = [&](int nb, uint4(&d)[STEPS]) {
      const int j0 = wave_first + nb * 64;
      const int boff = j0 * row_bytes + lane_off;
      if (ALL || j0 + 64 <= T) {
#pragma unroll
        for (int t = 0; t < STEPS; ++t) d[t] = ld16(rk, boff, t * step_bytes);
      } else {
        // ragged tail: slots at or past T read an in-range row; their sums feed unstored scores
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
          const bool in = j0 + t * KPS + kk < T;
          d[t] = ld16(rk, in ? boff + t * step_bytes : piece, 0);
        }
      }
    };
    // Batch 1 goes out with batch 0, before the set-up arithmetic -- except with the norm term,
    // whose set-up holds more registers: issued first there, its loads push the kernel past 256
    // registers and to one wave per SIMD, so it goes out after the set-up.
    constexpr bool EARLY_B1 = NB > 1 && !NORM;
    __builtin_amdgcn_sched_barrier(0);
    uint4 da[STEPS], db[STEPS];
    issue(0, da);
    if (EARLY_B1) issue(1, db);
    __builtin_amdgcn_sched_barrier(0);

    float2 v[BPL], w[BPL];
    float cn[BPL];
    const double m0 = tq - static_cast<double>(wave_first + kk);
#pragma unroll
    for (int i = 0; i < BPL; ++i) {
      if (live) {
        const double rev = rv[i];
        w[i] = cis_rev(rev, -static_cast<double>(KPS));
        v[i] = cmul(cmul(qv[i], av[i]), cis_rev(rev, m0));
        cn[i] = NORM ? norm_weight_of(qa[i], qv[i]) : 0.f;
      } else {
        w[i] = make_float2(1.f, 0.f);
        v[i] = make_float2(0.f, 0.f);
        cn[i] = 0.f;
      }
    }

    auto consume = [&](int nb, const uint4(&d)[STEPS]) {
      float acc[STEPS];
#pragma unroll
      for (int t = 0; t < STEPS; ++t) {
        const float a = lane_dot<BF16, NORM>(d[t], v, cn);
        acc[t] = FULL ? a : (live ? a : 0.f);
#pragma unroll
        for (int i = 0; i < BPL; ++i) v[i] = cmul(v[i], w[i]);
      }
      const float sc = reduce_scatter<STEPS>(acc, g);
      const int jj = wave_first + nb * 64 + g * KPS + kk;
      if (jj < T) st_score(p.scores + slot0 + jj, sc);
    };

    if (NB > 1 && !EARLY_B1) {
      __builtin_amdgcn_sched_barrier(0);
      issue(1, db);
      __builtin_amdgcn_sched_barrier(0);
    }
    // The next batch is issued whether or not it holds live slots (a batch past T takes the ragged
    // path and reads in-range rows whose sums are not stored): with a load that is always issued,
    // each wait counts only the older batch, where a conditional issue made the compiler wait for
    // every load in flight before the first batch's arithmetic.
#pragma unroll
    for (int nb = 0; nb < NB; nb += 2) {
      if (nb >= nbat) break;
      if (nb > 0 && nb + 1 < NB) issue(nb + 1, db);   // batch 1 is already out
      consume(nb, da);
      if (nb + 1 >= nbat) break;
      if (nb + 2 < NB) issue(nb + 2, da);
      consume(nb + 1, db);
    }
  };
  // With the norm term the branch-free copy lets the scheduler hold more than 256 registers (one
  // wave per SIMD, 35 % slower), so that form keeps the per-batch test.
  if (!NORM && wave_first + NB * 64 <= T) body(std::true_type{});
  else body(std::false_type{});
}

template <bool BF16, bool POS, bool FULL, bool NORM>
hipError_t launch_lpk(const ScoreParams &p, int lpk, dim3 grid, hipStream_t st) {
  const dim3 blk(kScoreThreads);
  if (!POS && KV_SCORE_PIPELINE) {
    switch (lpk) {
      case 1: hipLaunchKernelGGL((score_stream_kernel<BF16, 1, FULL, NORM>), grid, blk, 0, st, p); return hipGetLastError();
      case 2: hipLaunchKernelGGL((score_stream_kernel<BF16, 2, FULL, NORM>), grid, blk, 0, st, p); return hipGetLastError();
      case 4: hipLaunchKernelGGL((score_stream_kernel<BF16, 4, FULL, NORM>), grid, blk, 0, st, p); return hipGetLastError();
      case 8: hipLaunchKernelGGL((score_stream_kernel<BF16, 8, FULL, NORM>), grid, blk, 0, st, p); return hipGetLastError();
      case 16: hipLaunchKernelGGL((score_stream_kernel<BF16, 16, FULL, NORM>), grid, blk, 0, st, p); return hipGetLastError();
      default: break;
    }
  }
  switch (lpk) {
    case 1: hipLaunchKernelGGL((score_kernel<BF16, 1, POS, FULL, NORM>), grid, blk, 0, st, p); break;
    case 2: hipLaunchKernelGGL((score_kernel<BF16, 2, POS, FULL, NORM>), grid, blk, 0, st, p); break;
    case 4: hipLaunchKernelGGL((score_kernel<BF16, 4, POS, FULL, NORM>), grid, blk, 0, st, p); break;
    case 8: hipLaunchKernelGGL((score_kernel<BF16, 8, POS, FULL, NORM>), grid, blk, 0, st, p); break;
    case 16: hipLaunchKernelGGL((score_kernel<BF16, 16, POS, FULL, NORM>), grid, blk, 0, st, p); break;
    case 32: hipLaunchKernelGGL((score_kernel<BF16, 32, POS, FULL, NORM>), grid, blk, 0, st, p); break;
    case 64:  // only fp32 rows reach 64 pieces (head_dim 256)
      if constexpr (BF16) return hipErrorInvalidValue;
      else hipLaunchKernelGGL((score_kernel<BF16, 64, POS, FULL, NORM>), grid, blk, 0, st, p);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16, bool POS>
hipError_t launch_full(const ScoreParams &p, int lpk, dim3 grid, hipStream_t st) {
  const int bpl = BF16 ? 4 : 2;
  const bool full = lpk * bpl == p.F;
  if (p.qabs) return full ? launch_lpk<BF16, POS, true, true>(p, lpk, grid, st)
                          : launch_lpk<BF16, POS, false, true>(p, lpk, grid, st);
  return full ? launch_lpk<BF16, POS, true, false>(p, lpk, grid, st)
              : launch_lpk<BF16, POS, false, false>(p, lpk, grid, st);
}

}  // namespace

hipError_t launch_score(const ScoreParams &p, int dtype_bf16, int lanes_per_key, hipStream_t st) {
  const long long blocks = static_cast<long long>(p.L) * p.S * p.H * p.chunks_per_head;
  if (blocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(blocks));
  const bool pos = p.pos != nullptr;
  if (dtype_bf16) return pos ? launch_full<true, true>(p, lanes_per_key, grid, st)
                             : launch_full<true, false>(p, lanes_per_key, grid, st);
  return pos ? launch_full<false, true>(p, lanes_per_key, grid, st)
             : launch_full<false, false>(p, lanes_per_key, grid, st);
}

}  // namespace kvevict

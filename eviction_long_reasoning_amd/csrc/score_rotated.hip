// Key scores for keys stored after RoPE, dense or paged, for gfx950.
//
// What is computed: the same offset-averaged query-centre score as the
// pre-RoPE kernel ("TriAttention: Efficient Long Reasoning with Trigonometric
// KV Compression", structured summary 3.4, "The Trigonometric Series Term",
// "Handling Multiple Future Positions"), for keys a serving engine already
// stores rotated (the blog walkthrough's implementation scores the rotated
// key directly). With k_rot = RoPE(k, p) the key's own rotation cancels and
//
//   S_j = sum_f Re( W_f * conj(k_rot_{j,f}) ),   W_f = q_bar_f * A_f * exp(i omega_f t)
//
// so every key of a (layer, sequence, head) is dotted with one fixed vector:
// no per-key phase at all. Written out in the storage layout, W becomes a
// real weight per coordinate (the real part of W_f where band f's real part
// is stored, the imaginary part where its imaginary part is stored), for the
// interleaved (x[2f], x[2f+1]) or the half-split (x[f], x[f+d/2]) pairing.
//
// Keys come from a dense [L,S,H,t_cap,d] tensor or from a paged pool through a per-sequence
// block table, token-major [L, n_blocks, block_size, H, d] or head-major
// [L, n_blocks, H, block_size, d]. Lane layout, batching and the shuffle reduce-scatter follow
// the pre-RoPE kernel.
#include "kv_internal.hpp"
#include "rot_rows.hpp"

#ifndef KV_ROT_PREFETCH
#define KV_ROT_PREFETCH 1
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

template <int N>
__device__ __forceinline__ float reduce_scatter(float (&acc)[N], int g) {
#pragma unroll
  for (int h = N / 2; h >= 1; h /= 2) {
    const bool upper = (g & h) != 0;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      float lo = acc[i], hi = acc[i + h];
      asm volatile("" : "+v"(lo), "+v"(hi));  // keep the per-lane choice a register select
      const float send = upper ? lo : hi;
      const float keep = upper ? hi : lo;
      acc[i] = keep + __shfl_xor(send, h, 64);
    }
  }
  return acc[0];
}

typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const char *p) {
  const v4u32 v = __builtin_nontemporal_load(reinterpret_cast<const v4u32 *>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <bool BF16>
__device__ __forceinline__ float elem(const uint4 &d, int e) {
  const uint32_t wd[4] = {d.x, d.y, d.z, d.w};
  if (BF16) return __uint_as_float((e & 1) ? (wd[e >> 1] & 0xffff0000u) : (wd[e >> 1] << 16));
  return __uint_as_float(wd[e]);
}

// BF16: 8 coordinates per 16-byte lane piece (fp32: 4). HALF: half-split pairing. LAYOUT: 0 dense,
// 1 token-major paged pool, 2 head-major paged pool. NORM: add (1 - R_f) E|q_f| |k_f|.
template <bool BF16, int LPK, bool HALF, int LAYOUT, bool NORM>
__global__ __launch_bounds__(kScoreThreads) void score_rotated_kernel(const RotScoreParams p) {
  constexpr bool PAGED = LAYOUT != 0;
  constexpr int EPL = BF16 ? 8 : 4;            // coordinates per lane
  constexpr int KPS = 64 / LPK;
  constexpr int STEPS = LPK;
  constexpr int SUB = STEPS < 16 ? STEPS : 16;
  constexpr int EB = BF16 ? 2 : 4;

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
  const int wave_first = chunk * kScoreChunk + wave * (kScoreBatchesPerWave * 64);
  if (wave_first >= T) return;

  RowSpace rs;
  rs.K = static_cast<const char *>(p.K);
  rs.row_bytes = static_cast<int64_t>(p.d) * EB;
  rs.first = static_cast<int64_t>(head) * p.t_cap;
  rs.blk0 = static_cast<int64_t>(l) * p.n_blocks;
  rs.H = p.H;
  rs.h = h;
  rs.shift = p.block_shift;
  rs.n_blocks = p.n_blocks;
  rs.table = PAGED ? p.block_table + static_cast<size_t>(s) * p.blocks_per_seq : nullptr;
  const bool uni = uniform_steps<LAYOUT, KPS>(rs);
  const bool live = g * EPL < p.d;
  const int lane_off = live ? static_cast<int>(kk * slot_stride<LAYOUT>(rs)) + g * 16 : kRowOffIdle;

  // Block-table entries of the wave's slots, read before the weight set-up so that their latency
  // overlaps it (measured 4-7 % faster on shuffled paged pools; KV_ROT_PREFETCH=0 reads each
  // entry just before its row, as the dense path does): one id per block and batch when steps
  // share a block, else one per slot
  int ents[PAGED ? kScoreBatchesPerWave : 1];
  if constexpr (PAGED) {
    if (uni) {
#pragma unroll
      for (int nb = 0; nb < kScoreBatchesPerWave; ++nb) {
        const int j0 = wave_first + nb * 64;
        ents[nb] = step_entry<KPS>(rs, j0 < T ? j0 : 0, T, lane);
      }
    }
  }
  constexpr bool PREFETCH = PAGED && KV_ROT_PREFETCH && STEPS <= 16;
  int pbs[PREFETCH ? kScoreBatchesPerWave : 1][PREFETCH ? STEPS : 1];
  if constexpr (PREFETCH) {
    if (!uni) {
      const int32_t *tb = p.block_table + static_cast<size_t>(s) * p.blocks_per_seq;
#pragma unroll
      for (int nb = 0; nb < kScoreBatchesPerWave; ++nb) {
#pragma unroll
        for (int t = 0; t < STEPS; ++t) {
          int j = wave_first + nb * 64 + t * KPS + kk;
          j = j < T ? j : 0;
          pbs[nb][t] = min(max(tb[j >> p.block_shift], 0), p.n_blocks - 1);
        }
      }
    }
  }

  // per-coordinate weights of this lane's piece
  const int F = p.F;
  const size_t lh = static_cast<size_t>(l) * p.H + h;
  const float *q = p.qbar + lh * p.d;
  const double tq = static_cast<double>(p.t_cur[s]);
  float wgt[EPL];
  float cn[EPL];  // norm weight of the band owned by coordinate e (applied once per band)
  if constexpr (PAGED) {
    // Paged pools: the inputs of every coordinate are read first (an idle coordinate reads band 0)
    // and only then combined, so the reads overlap instead of each waiting for the one before
    // (shuffled 16-slot pool 3.25 -> 3.20 ms; dense heads, whose first rows arrive sooner, measured
    // 1.6 % slower this way and keep the loop below).
    float2 qfs[EPL], As[EPL];
    double revs[EPL];
    float qas[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int x = g * EPL + e;
      const bool valid = live && x < p.d;
      const int f = !valid ? 0 : (HALF ? (x < F ? x : x - F) : (x >> 1));
      qfs[e] = HALF ? make_float2(q[f], q[f + F]) : make_float2(q[2 * f], q[2 * f + 1]);
      As[e] = p.A[f];
      revs[e] = p.rev[f];
      qas[e] = NORM ? p.qabs[lh * F + f] : 0.f;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int x = g * EPL + e;
      wgt[e] = 0.f;
      cn[e] = 0.f;
      if (!live || x >= p.d) continue;
      const bool is_re = HALF ? (x < F) : ((x & 1) == 0);
      const float2 qf = qfs[e];
      const float2 W = cmul(cmul(qf, As[e]), cis_rev(revs[e], tq));
      wgt[e] = is_re ? W.x : W.y;
      if (NORM && is_re) cn[e] = qas[e] > 0.f ? qas[e] - sqrtf(fmaf(qf.x, qf.x, qf.y * qf.y)) : 0.f;
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int x = g * EPL + e;
      wgt[e] = 0.f;
      cn[e] = 0.f;
      if (!live || x >= p.d) continue;
      const int f = HALF ? (x < F ? x : x - F) : (x >> 1);
      const bool is_re = HALF ? (x < F) : ((x & 1) == 0);
      const float2 qf = HALF ? make_float2(q[f], q[f + F]) : make_float2(q[2 * f], q[2 * f + 1]);
      const float2 W = cmul(cmul(qf, p.A[f]), cis_rev(p.rev[f], tq));
      wgt[e] = is_re ? W.x : W.y;
      if (NORM && is_re) {
        const float qa = p.qabs[lh * F + f];
        cn[e] = qa > 0.f ? qa - sqrtf(fmaf(qf.x, qf.x, qf.y * qf.y)) : 0.f;
      }
    }
  }

  const size_t row_bytes = static_cast<size_t>(p.d) * EB;
  const char *Kb = static_cast<const char *>(p.K);
  const size_t dense0 = static_cast<size_t>(head) * p.t_cap;
  const int32_t *table = PAGED ? p.block_table + static_cast<size_t>(s) * p.blocks_per_seq : nullptr;
  const int bmask = (1 << p.block_shift) - 1;
  auto row_ptr = [&](int j, int pre) -> const char * {
    size_t row;
    if (PAGED) {
      int pb = PREFETCH ? pre : table[j >> p.block_shift];
      pb = min(max(pb, 0), p.n_blocks - 1);  // never leave the pool
      const size_t blk = static_cast<size_t>(l) * p.n_blocks + pb;
      row = LAYOUT == 2 ? (blk * p.H + h) * (bmask + 1) + (j & bmask) : (blk * (bmask + 1) + (j & bmask)) * p.H + h;
    } else {
      row = dense0 + j;
    }
    return Kb + row * row_bytes + static_cast<size_t>(live ? g : 0) * 16;
  };

#pragma unroll
  for (int nb = 0; nb < kScoreBatchesPerWave; ++nb) {
    const int j0 = wave_first + nb * 64;
    if (j0 >= T) break;
    float acc[STEPS];
    BatchSteps steps{};
    if (uni) steps = batch_steps<LAYOUT, KPS>(rs, j0, T, lane, PAGED ? ents[PAGED ? nb : 0] : 0);
#pragma unroll
    for (int st0 = 0; st0 < STEPS; st0 += SUB) {
      uint4 data[SUB];
#pragma unroll
      for (int t = 0; t < SUB; ++t) {
        if (uni) {
          data[t] = load_row_piece(step_rsrc(steps, st0 + t), lane_off);
        } else {
          const int j = j0 + (st0 + t) * KPS + kk;
          int pre = 0;
          if constexpr (PREFETCH) pre = pbs[nb][st0 + t];
          data[t] = ld_stream(row_ptr(j < T ? j : 0, pre));  // slots past T read row 0; their sums are not stored
        }
      }
#pragma unroll
      for (int t = 0; t < SUB; ++t) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) a = fmaf(wgt[e], elem<BF16>(data[t], e), a);
        if (NORM) {
          if (HALF) {
            // band f's two coordinates sit in lanes g and g ^ LPK/2; the lower lane adds the term
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
              const float v = elem<BF16>(data[t], e);
              const float other = __shfl_xor(v, LPK / 2, 64);
              a = fmaf(cn[e], __builtin_amdgcn_sqrtf(fmaf(v, v, other * other)), a);
            }
          } else {
#pragma unroll
            for (int e = 0; e < EPL; e += 2) {
              const float re = elem<BF16>(data[t], e), im = elem<BF16>(data[t], e + 1);
              a = fmaf(cn[e], __builtin_amdgcn_sqrtf(fmaf(re, re, im * im)), a);
            }
          }
        }
        acc[st0 + t] = a;
      }
    }
    if (!uni && !live) {   // per-slot rows: idle lanes read a live piece (uniform rows read zeros there)
#pragma unroll
      for (int t = 0; t < STEPS; ++t) acc[t] = 0.f;
    }
    const float sc = reduce_scatter<STEPS>(acc, g);
    const int jj = j0 + g * KPS + kk;
    if (jj < T) __builtin_nontemporal_store(sc, p.scores + dense0 + jj);
  }
}

template <bool BF16, bool HALF, int LAYOUT, bool NORM>
hipError_t launch_rot(const RotScoreParams &p, int lpk, dim3 grid, hipStream_t st) {
  const dim3 blk(kScoreThreads);
  switch (lpk) {
    case 1: hipLaunchKernelGGL((score_rotated_kernel<BF16, 1, HALF, LAYOUT, NORM>), grid, blk, 0, st, p); break;
    case 2: hipLaunchKernelGGL((score_rotated_kernel<BF16, 2, HALF, LAYOUT, NORM>), grid, blk, 0, st, p); break;
    case 4: hipLaunchKernelGGL((score_rotated_kernel<BF16, 4, HALF, LAYOUT, NORM>), grid, blk, 0, st, p); break;
    case 8: hipLaunchKernelGGL((score_rotated_kernel<BF16, 8, HALF, LAYOUT, NORM>), grid, blk, 0, st, p); break;
    case 16: hipLaunchKernelGGL((score_rotated_kernel<BF16, 16, HALF, LAYOUT, NORM>), grid, blk, 0, st, p); break;
    case 32: hipLaunchKernelGGL((score_rotated_kernel<BF16, 32, HALF, LAYOUT, NORM>), grid, blk, 0, st, p); break;
    case 64:  // only fp32 rows reach 64 pieces (head_dim 256)
      if constexpr (BF16) return hipErrorInvalidValue;
      else hipLaunchKernelGGL((score_rotated_kernel<BF16, 64, HALF, LAYOUT, NORM>), grid, blk, 0, st, p);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16, bool HALF, int LAYOUT>
hipError_t launch_rot_norm(const RotScoreParams &p, int lpk, dim3 grid, hipStream_t st) {
  return p.qabs != nullptr ? launch_rot<BF16, HALF, LAYOUT, true>(p, lpk, grid, st)
                           : launch_rot<BF16, HALF, LAYOUT, false>(p, lpk, grid, st);
}

template <bool BF16, bool HALF>
hipError_t launch_rot_flags(const RotScoreParams &p, int lpk, dim3 grid, hipStream_t st) {
  if (p.block_table == nullptr) return launch_rot_norm<BF16, HALF, 0>(p, lpk, grid, st);
  return p.head_major ? launch_rot_norm<BF16, HALF, 2>(p, lpk, grid, st)
                      : launch_rot_norm<BF16, HALF, 1>(p, lpk, grid, st);
}

}  // namespace

hipError_t launch_score_rotated(const RotScoreParams &p, int dtype_bf16, int lanes_per_key, hipStream_t st) {
  const long long blocks = static_cast<long long>(p.L) * p.S * p.H * p.chunks_per_head;
  if (blocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (dtype_bf16) return p.half ? launch_rot_flags<true, true>(p, lanes_per_key, grid, st)
                                : launch_rot_flags<true, false>(p, lanes_per_key, grid, st);
  return p.half ? launch_rot_flags<false, true>(p, lanes_per_key, grid, st)
                : launch_rot_flags<false, false>(p, lanes_per_key, grid, st);
}

}  // namespace kvevict

// Grouped-query scores: per-query-head scores, z-normalised per query head, max over the group.
//
// What is computed: "TriAttention: Efficient Long Reasoning with Trigonometric
// KV Compression" (structured summary 3.4, "KV Cache Pruning Procedure", the
// GQA handling): each of the G query heads sharing a KV head scores every
// cached key with its own centre, its scores are normalised to zero mean and
// unit (population) standard deviation over the head's T cached keys, and the
// key's final score is the maximum of its G normalised scores.
//
// The G dot products of a key are a dense contraction: for a tile of 16 keys, Y (16 keys x the 2F
// real coordinates of y_f = exp(i omega_f m) conj(k_f), m = t - p) times U (2F x G, the real and
// imaginary parts of u_{g,f} = q_bar_{g,f} A_f), since Re(u y) = u.x y.x - u.y y.y. Kernel A
// runs it on the matrix cores with v_mfma_f32_16x16x4_f32: lane l holds key l % 16 of the tile
// and the coordinates of quarter l / 16 of its row (16-byte pieces q, q + 4, q + 8, ... so each
// load instruction reads 64 contiguous bytes of 16 rows), forms y on the VALU (one complex
// product per band, the phase advanced by a fixed rotation per tile, or derived exactly per key
// for explicit positions) and feeds it as the A operand; the B operand is the same lane's slot
// of U for query head l % 16, and the four quarters are the MFMA's K = 4. Every coordinate of
// the tile is one MFMA and the product needs no cross-lane reduction: lane l ends up holding
// query head l % 16's scores of keys 4 (l / 16) .. + 3. Up to 16 query heads cost the same as
// one. The norm-based term is the same contraction over |k_f| and (E|q_f| - |q_bar_f|).
// Forming y costs as many VALU cycles per tile as the 32 MFMAs take, and the two were measured
// not to overlap; with at most four query heads 12 of the MFMA's 16 columns idle, and the VALU
// form (two FMAs per head and band on the y it forms anyway, gqa_stream_kernel) is faster. So
// groups of at most four with contiguous positions and bf16 rows of 4, 8 or 16 pieces take the
// VALU form; everything else the matrix form.
// Kernel A writes the G raw scores and, per (head, chunk of keys), fp64 sums of s and s^2 for
// each g. Kernel B reduces a head's chunk sums in a fixed order (deterministic, no atomics) and
// writes max_g (s_g - mu_g) / sigma_g (0 for a query head whose scores do not vary).
#include <type_traits>

#include "kv_internal.hpp"
#include "rot_rows.hpp"

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

typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Largest group scored by the VALU stream form (gqa_stream_kernel); 0 sends every group to the
// matrix cores
#ifndef KV_GQA_STREAM_MAX_G
#define KV_GQA_STREAM_MAX_G 4
#endif

constexpr int kTile = kGqaTile;
constexpr int kTilesPerWave = kGqaTilesPerWave;

// PPQ: 16-byte pieces per lane (pieces q, q + 4, ...); the row has p.d * e / 16 pieces, exactly
// 4 * PPQ of them when FULL. Up to PPQ = 4 the register budget is held to two waves per SIMD
// (one wave per SIMD measured 35 % slower).
template <bool BF16, int PPQ, bool FULL, bool POS, bool NORM>
__global__ __launch_bounds__(kScoreThreads, PPQ <= 4 ? 2 : 1) void score_gqa_kernel(const GqaParams p) {
  constexpr int BPL = BF16 ? 4 : 2;   // bands per piece
  constexpr int NB = PPQ * BPL;       // bands per lane
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int NW = kScoreThreads / 64;
  __shared__ double part[NW][16][2];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = lane & 15;          // A: key of the tile; B and D: query head
  const int q = lane >> 4;            // quarter of the row (the MFMA's K index)
  const int head = blockIdx.x / p.chunks_per_head;
  const int chunk = blockIdx.x - head * p.chunks_per_head;
  const int h = head % p.H;
  const int s = (head / p.H) % p.S;
  const int l = head / (p.H * p.S);
  const int G = p.G;

  const int T = min(max(p.seq_len[s], 0), p.t_cap);
  const int wave_first = chunk * kGqaChunk + wave * (kTilesPerWave * kTile);
  const double tq = static_cast<double>(p.t_cur[s]);
  const int pieces = FULL ? 4 * PPQ : p.d * EB / 16;

  // this lane's slot of U (query head `row`) and its bands' phase constants
  float ux[NB], uy[NB], cn[NB];
  double rev[NB];
  const size_t lhg = (static_cast<size_t>(l) * p.H + h) * G;
#pragma unroll
  for (int m = 0; m < PPQ; ++m) {
#pragma unroll
    for (int c = 0; c < BPL; ++c) {
      const int n = m * BPL + c;
      const int pc = q + 4 * m;
      const int f = pc * BPL + c;
      const bool live = FULL || pc < pieces;
      rev[n] = live ? p.rev[f] : 0.0;
      ux[n] = uy[n] = cn[n] = 0.f;
      if (live && row < G) {
        const float2 qf = reinterpret_cast<const float2 *>(p.qbar + (lhg + row) * p.d)[f];
        const float2 A = p.A[f];
        ux[n] = qf.x * A.x - qf.y * A.y;
        uy[n] = -(qf.x * A.y + qf.y * A.x);          // Re(u y) = u.x y.x + (-u.y) y.y
        if (NORM) {
          const float qa = p.qabs[(lhg + row) * p.F + f];
          cn[n] = qa > 0.f ? qa - __builtin_amdgcn_sqrtf(fmaf(qf.x, qf.x, qf.y * qf.y)) : 0.f;
        }
      }
    }
  }
  double sum = 0.0, sum2 = 0.0;

  const size_t slot0 = static_cast<size_t>(head) * p.t_cap;
  const size_t row_bytes = static_cast<size_t>(p.d) * EB;
  const char *Kh = static_cast<const char *>(p.K) + slot0 * row_bytes;
  float2 z[NB], w[NB];
  if (!POS && wave_first < T) {
    const double m0 = tq - static_cast<double>(wave_first + row);
#pragma unroll
    for (int m = 0; m < PPQ; ++m) {
#pragma unroll
      for (int c = 0; c < BPL; ++c) {
        const int n = m * BPL + c;
        const int pc = q + 4 * m;
        z[n] = cis_rev(rev[n], m0);
        w[n] = (FULL || pc < pieces) ? p.W[pc * BPL + c] : make_float2(1.f, 0.f);
      }
    }
  }
  auto load_tile = [&](int j0, uint4 (&d)[PPQ], int32_t &pj) {
    const int j = j0 + row;
    const int jc = j < T ? j : T - 1;   // slots past T repeat the last row; their scores are not kept
    const char *r = Kh + static_cast<size_t>(jc) * row_bytes;
#pragma unroll
    for (int m = 0; m < PPQ; ++m) {
      const int pc = q + 4 * m;
      if (FULL || pc < pieces) {
        const v4u32 v = __builtin_nontemporal_load(reinterpret_cast<const v4u32 *>(r + pc * 16));
        d[m] = make_uint4(v[0], v[1], v[2], v[3]);
      } else {
        d[m] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    if (POS) pj = p.pos[slot0 + jc];
  };

  // Tiles in flight: tile t + AHEAD loads while tile t is computed. The buffers shift down one
  // slot per tile; fully unrolled, the shifts are register renames. With explicit positions each
  // tile's phases are derived during the tile before it, from a position loaded two tiles ahead
  // (one ahead from four pieces per lane on, where the registers would cost a wave per SIMD).
  // The VALU and the matrix cores do not run at the same time on this part (the SQ counter of
  // cycles with both busy reads 0), so this gains only what the smaller live range saves.
  constexpr int AHEAD = POS ? (PPQ <= 2 ? 2 : 1) : (PPQ > 4 ? 1 : 3);
  uint4 buf[AHEAD + 1][PPQ];
  int32_t pbuf[AHEAD + 1] = {};   // a tile past the wave's last one keeps position 0 (its phases go unused)
#pragma unroll
  for (int a = 0; a < AHEAD; ++a)
    if (wave_first + a * kTile < T) load_tile(wave_first + a * kTile, buf[a], pbuf[a]);

  // Explicit positions, two tiles ahead: the first tile's phases here; each later tile's are
  // derived during the tile before it (tile_scores' pnext), after that tile's products are issued.
  // One tile ahead, each tile derives its own phases first (its position has had longest to arrive).
  constexpr bool PIPE = POS && AHEAD == 2;
  if (PIPE && wave_first < T) {
    const double m = tq - static_cast<double>(pbuf[0]);
#pragma unroll
    for (int n = 0; n < NB; ++n) z[n] = cis_rev(rev[n], m);
  }

  // one tile: y on the VALU, the contraction on the matrix cores; then the next tile's phases
  // (explicit positions two tiles ahead: from pnext) or the fixed rotation to the next tile
  auto tile_scores = [&](const uint4 (&cur)[PPQ], int32_t pcur, int32_t pnext) -> v4f {
    if (POS && !PIPE) {
      const double m = tq - static_cast<double>(pcur);
#pragma unroll
      for (int n = 0; n < NB; ++n) z[n] = cis_rev(rev[n], m);
    }
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < PPQ; ++m) {
      const uint32_t wd[4] = {cur[m].x, cur[m].y, cur[m].z, cur[m].w};
#pragma unroll
      for (int c = 0; c < BPL; ++c) {
        const int n = m * BPL + c;
        const float re = BF16 ? __uint_as_float(wd[c] << 16) : __uint_as_float(wd[2 * c]);
        const float im = BF16 ? __uint_as_float(wd[c] & 0xffff0000u) : __uint_as_float(wd[2 * c + 1]);
        const float yx = fmaf(z[n].x, re, z[n].y * im);    // y = z conj(k)
        const float yy = fmaf(z[n].y, re, -z[n].x * im);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(yx, ux[n], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(yy, uy[n], acc, 0, 0, 0);
        if (NORM) {
          const float ka = __builtin_amdgcn_sqrtf(fmaf(re, re, im * im));
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka, cn[n], acc, 0, 0, 0);
        }
      }
    }
    if (PIPE) {
      const double m = tq - static_cast<double>(pnext);
#pragma unroll
      for (int n = 0; n < NB; ++n) z[n] = cis_rev(rev[n], m);
    } else if (!POS) {
#pragma unroll
      for (int n = 0; n < NB; ++n) z[n] = cmul(z[n], w[n]);
    }
    return acc;
  };
  auto next_tile = [&](int t, int j0, uint4 (&cur)[PPQ], int32_t &pcur) {
    if (t + AHEAD < kTilesPerWave && j0 + AHEAD * kTile < T) load_tile(j0 + AHEAD * kTile, buf[AHEAD], pbuf[AHEAD]);
#pragma unroll
    for (int m = 0; m < PPQ; ++m) cur[m] = buf[0][m];
    pcur = pbuf[0];
#pragma unroll
    for (int a = 0; a < AHEAD; ++a) {
#pragma unroll
      for (int m = 0; m < PPQ; ++m) buf[a][m] = buf[a + 1][m];
      pbuf[a] = pbuf[a + 1];
    }
  };

  // lane holds query head `row`'s scores of keys j0 + 4q .. + 3; a query head row >= G has all
  // zero scores and is not stored
  float *raw_head = p.raw + static_cast<size_t>(head) * G * p.t_cap;
  if (wave_first + kTilesPerWave * kTile <= T) {
    // every tile of the wave is full: a branch-free body, stored through a buffer resource whose
    // bounds drop the stores of rows >= G
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
        raw_head, 0, static_cast<int>(static_cast<size_t>(G) * p.t_cap * 4), 0x00020000);
    const int row_off = row < G ? row * p.t_cap * 4 : 0x7FFFFFF0;
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      const int j0 = wave_first + t * kTile;
      uint4 cur[PPQ];
      int32_t pcur;
      next_tile(t, j0, cur, pcur);
      const v4f acc = tile_scores(cur, pcur, pbuf[0]);
      const v4u32 bits = {__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                          __float_as_uint(acc[3])};
      __builtin_amdgcn_raw_buffer_store_b128(bits, rr, row_off + (j0 + 4 * q) * 4, 0, 2);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sum += static_cast<double>(acc[r]);
        sum2 += static_cast<double>(acc[r]) * static_cast<double>(acc[r]);
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < kTilesPerWave; ++t) {
      const int j0 = wave_first + t * kTile;
      if (j0 >= T) break;
      uint4 cur[PPQ];
      int32_t pcur;
      next_tile(t, j0, cur, pcur);
      const v4f acc = tile_scores(cur, pcur, pbuf[0]);
      const int jk = j0 + 4 * q;
      if (row < G) {
        float *dst = raw_head + static_cast<size_t>(row) * p.t_cap + jk;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (jk + r < T) {
            const float sc = acc[r];
            __builtin_nontemporal_store(sc, dst + r);
            sum += static_cast<double>(sc);
            sum2 += static_cast<double>(sc) * static_cast<double>(sc);
          }
        }
      }
    }
  }
  // per (head, chunk) sums for each query head, in a fixed reduction order
  sum += __shfl_xor(sum, 16, 64);
  sum2 += __shfl_xor(sum2, 16, 64);
  sum += __shfl_xor(sum, 32, 64);
  sum2 += __shfl_xor(sum2, 32, 64);
  if (q == 0) {
    part[wave][row][0] = sum;
    part[wave][row][1] = sum2;
  }
  __syncthreads();
  if (static_cast<int>(threadIdx.x) < G) {
    const int g = threadIdx.x;
    double a = 0.0, b = 0.0;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) {
      a += part[wv][g][0];
      b += part[wv][g][1];
    }
    double *dst = p.partials + ((static_cast<size_t>(head) * p.chunks_per_head + chunk) * G + g) * 2;
    dst[0] = a;
    dst[1] = b;
  }
}

// One workgroup per (head, chunk): reduce the head's chunk sums, then normalise and take the max.
template <int GM>
__global__ __launch_bounds__(kScoreThreads) void gqa_finish_kernel(const GqaParams p) {
  constexpr int NW = kScoreThreads / 64;
  constexpr int KPT = kGqaChunk / kScoreThreads;   // consecutive keys per thread
  static_assert(KPT == 4, "one float4 of keys per thread");
  __shared__ double stats[GM][2];  // mean, 1/std (0 when the std is 0)
  const int head = blockIdx.x / p.chunks_per_head;
  const int chunk = blockIdx.x - head * p.chunks_per_head;
  const int s = (head / p.H) % p.S;
  const int T = min(max(p.seq_len[s], 0), p.t_cap);
  const int j0 = chunk * kGqaChunk;
  if (j0 >= T) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the head's statistics, one query head per wave at a time (fixed summation order)
  const int n_chunks = (T + kGqaChunk - 1) / kGqaChunk;
  for (int g = wave; g < p.G; g += NW) {
    double a = 0.0, b = 0.0;
    for (int c = lane; c < n_chunks; c += 64) {
      const double *src = p.partials + ((static_cast<size_t>(head) * p.chunks_per_head + c) * p.G + g) * 2;
      a += src[0];
      b += src[1];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      a += __shfl_xor(a, off, 64);
      b += __shfl_xor(b, off, 64);
    }
    if (lane == 0) {
      const double mu = a / T;
      const double var = b / T - mu * mu;
      stats[g][0] = mu;
      stats[g][1] = var > 0.0 ? 1.0 / sqrt(var) : 0.0;
    }
  }
  __syncthreads();
  const int j = j0 + KPT * static_cast<int>(threadIdx.x);
  if (j >= T) return;
  const float *raw = p.raw + static_cast<size_t>(head) * p.G * p.t_cap + j;
  float *out = p.scores + static_cast<size_t>(head) * p.t_cap + j;
  const bool aligned = ((reinterpret_cast<uintptr_t>(p.raw) | reinterpret_cast<uintptr_t>(p.scores)) & 15u) == 0;
  if (aligned && (p.t_cap & 3) == 0 && j + KPT <= T) {
    v4f x[GM];
#pragma unroll
    for (int g = 0; g < GM; ++g)
      if (g < p.G) x[g] = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(raw + static_cast<size_t>(g) * p.t_cap));
    v4f best;
#pragma unroll
    for (int k = 0; k < KPT; ++k) {
      double m = -INFINITY;
#pragma unroll
      for (int g = 0; g < GM; ++g)
        if (g < p.G) m = fmax(m, (static_cast<double>(x[g][k]) - stats[g][0]) * stats[g][1]);
      best[k] = static_cast<float>(m);
    }
    __builtin_nontemporal_store(best, reinterpret_cast<v4f *>(out));
  } else {
    for (int k = 0; k < KPT && j + k < T; ++k) {
      double m = -INFINITY;
#pragma unroll
      for (int g = 0; g < GM; ++g)
        if (g < p.G) m = fmax(m, (static_cast<double>(raw[static_cast<size_t>(g) * p.t_cap + k]) - stats[g][0]) * stats[g][1]);
      out[k] = static_cast<float>(m);
    }
  }
}

// Small groups (G <= 4) with contiguous positions: the VALU form in the single-centre stream
// layout. LPK lanes share a key (one 16-byte piece each), KPS = 64 / LPK keys per wave load, the
// phase z = exp(i omega_f m) of a lane's key carried from key to key by a fixed step and derived
// exactly at every batch of 64 keys. Per band the lane forms y = z conj(k) once; each query head
// then costs two FMAs, Re(u_g y). Work goes in sub-batches of SUB = min(LPK, 8) steps whose loads
// are issued one sub-batch ahead (two register buffers); a sub-batch's SUB partial sums per query
// head are combined by a reduce-scatter over SUB lanes plus one exchange per further lane
// doubling, after which each lane of the first SUB of its key group holds one finished score.
// The fp64 sums of s and s^2 per (head, chunk) have the layout kernel B reads.
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

constexpr int kStreamLoadNt = 2;  // cache-policy bit "nt": every key row is read once
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStreamLoadNt);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Steps per sub-batch (at most): 4 was measured as fast as 8 (three waves per SIMD instead of two)
#ifndef KV_GQA_SUB
#define KV_GQA_SUB 8
#endif
template <bool BF16, int LPK, bool FULL, bool NORM, int GM>
__global__ __launch_bounds__(kScoreThreads) void gqa_stream_kernel(const GqaParams p) {
  constexpr int BPL = BF16 ? 4 : 2;
  constexpr int KPS = 64 / LPK;
  constexpr int SUB = LPK < KV_GQA_SUB ? LPK : KV_GQA_SUB;  // steps per sub-batch
  constexpr int SUB_KEYS = SUB * KPS;
  constexpr int NW = kScoreThreads / 64;
  constexpr int WAVE_KEYS = kGqaChunk / NW;
  constexpr int NSB = WAVE_KEYS / SUB_KEYS;       // sub-batches per wave
  constexpr int SB_PER_BATCH = 64 / SUB_KEYS;     // sub-batches per 64 keys (phase re-derived)
  constexpr int EB = BF16 ? 2 : 4;
  static_assert(WAVE_KEYS % 64 == 0 && NSB % 2 == 0, "whole batches, pairs of sub-batches");
  __shared__ double part[NW][GM][2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int g = lane % LPK;
  const int kk = lane / LPK;
  const int head = blockIdx.x / p.chunks_per_head;
  const int chunk = blockIdx.x - head * p.chunks_per_head;
  const int h = head % p.H;
  const int s = (head / p.H) % p.S;
  const int l = head / (p.H * p.S);
  const int G = p.G;

  const int T = min(max(p.seq_len[s], 0), p.t_cap);
  const int wave_first = chunk * kGqaChunk + wave * WAVE_KEYS;
  const int nsb = wave_first < T ? min(NSB, (T - wave_first + SUB_KEYS - 1) / SUB_KEYS) : 0;

  const bool live = FULL || g * BPL < p.F;
  const size_t slot0 = static_cast<size_t>(head) * p.t_cap;
  const int row_bytes = p.d * EB;
  // rows at or past T read as zeros (buffer range check); their scores are not stored
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char *>(static_cast<const char *>(p.K) + slot0 * static_cast<size_t>(row_bytes)), 0,
      T * row_bytes, 0x00020000);
  const int lane_off = kk * row_bytes + (live ? g * 16 : 0);
  const int step_bytes = KPS * row_bytes;
  auto issue = [&](int sb, uint4(&d)[SUB]) {
    const int boff = (wave_first + sb * SUB_KEYS) * row_bytes + lane_off;
#pragma unroll
    for (int t = 0; t < SUB; ++t) d[t] = ld16(rk, boff, t * step_bytes);
  };
  // Sub-batches are issued whether or not they hold live keys: past T the buffer range check
  // returns zeros without a memory access (offsets stay below 2^31: the launch requires
  // t_cap plus two chunks of rows to fit), and a load that is always issued lets each wait count only
  // the older sub-batch (a conditional issue forces a wait for every load in flight).
  uint4 da[SUB], db[SUB];
  issue(0, da);

  const double tq = static_cast<double>(p.t_cur[s]);
  const size_t lhg = (static_cast<size_t>(l) * p.H + h) * G;
  float ux[GM][BPL], uyn[GM][BPL], cn[GM][BPL];
  double rev[BPL];
  float2 w[BPL], z[BPL];
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const int b = g * BPL + i;
    rev[i] = live ? p.rev[b] : 0.0;
    w[i] = live ? cis_rev(rev[i], -static_cast<double>(KPS)) : make_float2(1.f, 0.f);
#pragma unroll
    for (int q = 0; q < GM; ++q) {
      ux[q][i] = uyn[q][i] = cn[q][i] = 0.f;
      if (live && q < G) {
        const float2 qf = reinterpret_cast<const float2 *>(p.qbar + (lhg + q) * p.d)[b];
        const float2 A = p.A[b];
        ux[q][i] = qf.x * A.x - qf.y * A.y;
        uyn[q][i] = -(qf.x * A.y + qf.y * A.x);       // Re(u y) = u.x y.x + (-u.y) y.y
        if (NORM) {
          const float qa = p.qabs[(lhg + q) * p.F + b];
          cn[q][i] = qa > 0.f ? qa - __builtin_amdgcn_sqrtf(fmaf(qf.x, qf.x, qf.y * qf.y)) : 0.f;
        }
      }
    }
  }
  double sum[GM], sum2[GM];
#pragma unroll
  for (int q = 0; q < GM; ++q) sum[q] = sum2[q] = 0.0;
  float *raw_head = p.raw + static_cast<size_t>(head) * G * p.t_cap;

  auto consume = [&](int sb, const uint4(&d)[SUB]) {
    const int j0 = wave_first + sb * SUB_KEYS;
    if (sb % SB_PER_BATCH == 0) {   // exact phase of this lane's first key of the batch
      const double m0 = tq - static_cast<double>(j0 + kk);
#pragma unroll
      for (int i = 0; i < BPL; ++i) z[i] = live ? cis_rev(rev[i], m0) : make_float2(0.f, 0.f);
    }
    float acc[GM][SUB];
#pragma unroll
    for (int t = 0; t < SUB; ++t) {
      const uint32_t wd[4] = {d[t].x, d[t].y, d[t].z, d[t].w};
      float a[GM];
#pragma unroll
      for (int q = 0; q < GM; ++q) a[q] = 0.f;
#pragma unroll
      for (int i = 0; i < BPL; ++i) {
        const float re = BF16 ? __uint_as_float(wd[i] << 16) : __uint_as_float(wd[2 * i]);
        const float im = BF16 ? __uint_as_float(wd[i] & 0xffff0000u) : __uint_as_float(wd[2 * i + 1]);
        const float yx = fmaf(z[i].x, re, z[i].y * im);    // y = z conj(k)
        const float yy = fmaf(z[i].y, re, -z[i].x * im);
        const float ka = NORM ? __builtin_amdgcn_sqrtf(fmaf(re, re, im * im)) : 0.f;
#pragma unroll
        for (int q = 0; q < GM; ++q) {
          a[q] = fmaf(ux[q][i], yx, a[q]);
          a[q] = fmaf(uyn[q][i], yy, a[q]);
          if (NORM) a[q] = fmaf(cn[q][i], ka, a[q]);
        }
      }
#pragma unroll
      for (int q = 0; q < GM; ++q) acc[q][t] = FULL ? a[q] : (live ? a[q] : 0.f);
#pragma unroll
      for (int i = 0; i < BPL; ++i) z[i] = cmul(z[i], w[i]);
    }
    const int jj = j0 + (g % SUB) * KPS + kk;
    const bool store = g < SUB && jj < T;
#pragma unroll
    for (int q = 0; q < GM; ++q) {
      float sc = reduce_scatter<SUB>(acc[q], g % SUB);
#pragma unroll
      for (int hh = SUB; hh < LPK; hh *= 2) sc += __shfl_xor(sc, hh, 64);
      if (store && q < G) {
        __builtin_nontemporal_store(sc, raw_head + static_cast<size_t>(q) * p.t_cap + jj);
        sum[q] += static_cast<double>(sc);
        sum2[q] += static_cast<double>(sc) * static_cast<double>(sc);
      }
    }
  };

#pragma unroll
  for (int sb = 0; sb < NSB; sb += 2) {
    if (sb >= nsb) break;
    issue(sb + 1, db);
    consume(sb, da);
    if (sb + 1 >= nsb) break;
    issue(sb + 2, da);
    consume(sb + 1, db);
  }

  // per (head, chunk) sums for each query head, in a fixed reduction order
#pragma unroll
  for (int q = 0; q < GM; ++q) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      sum[q] += __shfl_xor(sum[q], off, 64);
      sum2[q] += __shfl_xor(sum2[q], off, 64);
    }
    if (lane == 0) {
      part[wave][q][0] = sum[q];
      part[wave][q][1] = sum2[q];
    }
  }
  __syncthreads();
  if (static_cast<int>(threadIdx.x) < G) {
    const int q = threadIdx.x;
    double a = 0.0, b = 0.0;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) {
      a += part[wv][q][0];
      b += part[wv][q][1];
    }
    double *dst = p.partials + ((static_cast<size_t>(head) * p.chunks_per_head + chunk) * G + q) * 2;
    dst[0] = a;
    dst[1] = b;
  }
}

// Grouped-query scores of keys stored after RoPE, dense or paged (the serving layout). With
// k_rot = RoPE(k, p) a key's own rotation cancels, and query head g's score is one dot product with
// W_{g,f} = q_bar_{g,f} A_f exp(i omega_f t), written out per stored coordinate (the real part of
// W where band f's real part is stored, the imaginary part where its imaginary part is), for the
// interleaved or the half-split pairing. Lane layout (one 16-byte piece per lane, LPK lanes per
// key), the block-table addressing and the reduce-scatter follow the single-centre rotated
// kernel, with G accumulators per key; the raw scores and chunk sums have kernel A's layout, so
// kernel B is shared.
template <typename T>
__device__ __forceinline__ float coord(const uint4 &d, int e) {
  const uint32_t wd[4] = {d.x, d.y, d.z, d.w};
  if constexpr (sizeof(T) == 2) return __uint_as_float((e & 1) ? (wd[e >> 1] & 0xffff0000u) : (wd[e >> 1] << 16));
  else return __uint_as_float(wd[e]);
}

template <bool BF16, int LPK, bool HALF, int LAYOUT, bool NORM, int GM>
__global__ __launch_bounds__(kScoreThreads) void gqa_rotated_kernel(const GqaParams p) {
  constexpr bool PAGED = LAYOUT != 0;
  constexpr int EPL = BF16 ? 8 : 4;               // coordinates per lane (one 16-byte piece)
  constexpr int KPS = 64 / LPK;
  constexpr int STEPS = LPK;
  constexpr int NW = kScoreThreads / 64;
  constexpr int NB = kGqaChunk / NW / 64;         // 64-key batches per wave
  constexpr int EB = BF16 ? 2 : 4;
  using Elem = typename std::conditional<BF16, uint16_t, float>::type;
  __shared__ double part[NW][GM][2];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int g = lane % LPK;
  const int kk = lane / LPK;
  const int head = blockIdx.x / p.chunks_per_head;
  const int chunk = blockIdx.x - head * p.chunks_per_head;
  const int h = head % p.H;
  const int s = (head / p.H) % p.S;
  const int l = head / (p.H * p.S);
  const int G = p.G;
  const int F = p.F;

  const int T = min(max(p.seq_len[s], 0), p.t_cap);
  const int wave_first = chunk * kGqaChunk + wave * (NB * 64);
  const double tq = static_cast<double>(p.t_cur[s]);
  const bool live = g * EPL < p.d;
  const size_t lhg = (static_cast<size_t>(l) * p.H + h) * G;

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
  const int lane_off = live ? static_cast<int>(kk * slot_stride<LAYOUT>(rs)) + g * 16 : kRowOffIdle;
  // block-table entries of the next batch's steps (one per lane), read one batch ahead
  int ent_next = 0;
  if (PAGED && uni && wave_first < T) ent_next = step_entry<KPS>(rs, wave_first, T, lane);

  // per query head, the weight of each coordinate of this lane's piece (and the norm weight of the
  // band whose real part the coordinate holds)
  float wgt[GM][EPL], cn[GM][EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int x = g * EPL + e;
    const int f = HALF ? (x < F ? x : x - F) : (x >> 1);
    const bool is_re = HALF ? (x < F) : ((x & 1) == 0);
    float2 ph = make_float2(0.f, 0.f);
    if (live && x < p.d) ph = cmul(p.A[f], cis_rev(p.rev[f], tq));
#pragma unroll
    for (int q = 0; q < GM; ++q) {
      wgt[q][e] = cn[q][e] = 0.f;
      if (live && x < p.d && q < G) {
        const float *qg = p.qbar + (lhg + q) * p.d;
        const float2 qf = HALF ? make_float2(qg[f], qg[f + F]) : make_float2(qg[2 * f], qg[2 * f + 1]);
        const float2 W = cmul(qf, ph);
        wgt[q][e] = is_re ? W.x : W.y;
        if (NORM && is_re) {
          const float qa = p.qabs[(lhg + q) * F + f];
          cn[q][e] = qa > 0.f ? qa - __builtin_amdgcn_sqrtf(fmaf(qf.x, qf.x, qf.y * qf.y)) : 0.f;
        }
      }
    }
  }

  const size_t row_bytes = static_cast<size_t>(p.d) * EB;
  const char *Kb = static_cast<const char *>(p.K);
  const size_t dense0 = static_cast<size_t>(head) * p.t_cap;
  const int32_t *table = PAGED ? p.block_table + static_cast<size_t>(s) * p.blocks_per_seq : nullptr;
  const int bmask = (1 << p.block_shift) - 1;
  auto row_ptr = [&](int j) -> const char * {
    size_t row;
    if (PAGED) {
      const int pb = min(max(table[j >> p.block_shift], 0), p.n_blocks - 1);   // never leave the pool
      const size_t blk = static_cast<size_t>(l) * p.n_blocks + pb;
      row = LAYOUT == 2 ? (blk * p.H + h) * (bmask + 1) + (j & bmask) : (blk * (bmask + 1) + (j & bmask)) * p.H + h;
    } else {
      row = dense0 + j;
    }
    return Kb + row * row_bytes + static_cast<size_t>(live ? g : 0) * 16;
  };

  double sum[GM], sum2[GM];
#pragma unroll
  for (int q = 0; q < GM; ++q) sum[q] = sum2[q] = 0.0;
  float *raw_head = p.raw + static_cast<size_t>(head) * G * p.t_cap;

#pragma unroll 1
  for (int nb = 0; nb < NB; ++nb) {
    const int j0 = wave_first + nb * 64;
    if (j0 >= T) break;
    uint4 data[STEPS];
    if (uni) {
      const BatchSteps steps = batch_steps<LAYOUT, KPS>(rs, j0, T, lane, ent_next);
#pragma unroll
      for (int t = 0; t < STEPS; ++t) data[t] = load_row_piece(step_rsrc(steps, t), lane_off);
      if (PAGED && nb + 1 < NB && j0 + 64 < T) ent_next = step_entry<KPS>(rs, j0 + 64, T, lane);
      // all of the batch's loads go out before any of its arithmetic (left free, the scheduler
      // interleaves unpacking with the loads of dense heads and waits after every few)
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
      for (int t = 0; t < STEPS; ++t) {
        const int j = j0 + t * KPS + kk;
        const v4u32 v = __builtin_nontemporal_load(reinterpret_cast<const v4u32 *>(row_ptr(j < T ? j : 0)));
        data[t] = make_uint4(v[0], v[1], v[2], v[3]);   // slots past T read row 0; not stored
      }
    }
    float acc[GM][STEPS];
#pragma unroll
    for (int t = 0; t < STEPS; ++t) {
      float a[GM];
#pragma unroll
      for (int q = 0; q < GM; ++q) a[q] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float x = coord<Elem>(data[t], e);
#pragma unroll
        for (int q = 0; q < GM; ++q) a[q] = fmaf(wgt[q][e], x, a[q]);
        if (NORM) {
          float ka;
          if (HALF) {
            // band f's two coordinates sit in lanes g and g ^ LPK/2; the lower lane adds the term
            const float other = __shfl_xor(x, LPK / 2, 64);
            ka = __builtin_amdgcn_sqrtf(fmaf(x, x, other * other));
          } else {
            const float y = coord<Elem>(data[t], e ^ 1);
            ka = __builtin_amdgcn_sqrtf(fmaf(x, x, y * y));
          }
#pragma unroll
          for (int q = 0; q < GM; ++q) a[q] = fmaf(cn[q][e], ka, a[q]);
        }
      }
#pragma unroll
      for (int q = 0; q < GM; ++q) {
        acc[q][t] = a[q];
        // materialise every head's sum here: left free, the compiler sinks the dot products of
        // heads q >= 1 into the branches below and keeps the whole batch's keys in registers
        asm volatile("" : "+v"(acc[q][t]));
      }
      // one step at a time: unpacking a later piece early only holds more registers
      __builtin_amdgcn_sched_barrier(0);
    }
    if (!uni && !live) {   // per-slot rows: idle lanes read a live piece (uniform rows read zeros there)
#pragma unroll
      for (int q = 0; q < GM; ++q)
#pragma unroll
        for (int t = 0; t < STEPS; ++t) acc[q][t] = 0.f;
    }
    const int jj = j0 + g * KPS + kk;
#pragma unroll
    for (int q = 0; q < GM; ++q) {
      const float sc = reduce_scatter<STEPS>(acc[q], g);
      if (jj < T && q < G) {
        __builtin_nontemporal_store(sc, raw_head + static_cast<size_t>(q) * p.t_cap + jj);
        sum[q] += static_cast<double>(sc);
        sum2[q] += static_cast<double>(sc) * static_cast<double>(sc);
      }
    }
  }

  // per (head, chunk) sums for each query head, in a fixed reduction order
#pragma unroll
  for (int q = 0; q < GM; ++q) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      sum[q] += __shfl_xor(sum[q], off, 64);
      sum2[q] += __shfl_xor(sum2[q], off, 64);
    }
    if (lane == 0) {
      part[wave][q][0] = sum[q];
      part[wave][q][1] = sum2[q];
    }
  }
  __syncthreads();
  if (static_cast<int>(threadIdx.x) < G) {
    const int q = threadIdx.x;
    double a = 0.0, b = 0.0;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) {
      a += part[wv][q][0];
      b += part[wv][q][1];
    }
    double *dst = p.partials + ((static_cast<size_t>(head) * p.chunks_per_head + chunk) * G + q) * 2;
    dst[0] = a;
    dst[1] = b;
  }
}

int group_bound(int G) {
  int gm = 1;
  while (gm < G) gm <<= 1;
  return gm;
}

template <bool NORM, int GM>
hipError_t launch_stream_lpk(const GqaParams &p, int lpk, dim3 grid, hipStream_t st) {
  const dim3 blk(kScoreThreads);
  switch (lpk) {
    case 4: hipLaunchKernelGGL((gqa_stream_kernel<true, 4, true, NORM, GM>), grid, blk, 0, st, p); break;
    case 8: hipLaunchKernelGGL((gqa_stream_kernel<true, 8, true, NORM, GM>), grid, blk, 0, st, p); break;
    case 16: hipLaunchKernelGGL((gqa_stream_kernel<true, 16, true, NORM, GM>), grid, blk, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool NORM>
hipError_t launch_stream(const GqaParams &p, int lpk, dim3 grid, hipStream_t st) {
  switch (group_bound(p.G)) {
    case 1: return launch_stream_lpk<NORM, 1>(p, lpk, grid, st);
    case 2: return launch_stream_lpk<NORM, 2>(p, lpk, grid, st);
    case 4: return launch_stream_lpk<NORM, 4>(p, lpk, grid, st);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16, bool FULL, bool POS, bool NORM>
hipError_t launch_ppq(const GqaParams &p, int ppq, dim3 grid, hipStream_t st) {
  const dim3 blk(kScoreThreads);
  switch (ppq) {
    case 1: hipLaunchKernelGGL((score_gqa_kernel<BF16, 1, FULL, POS, NORM>), grid, blk, 0, st, p); break;
    case 2: hipLaunchKernelGGL((score_gqa_kernel<BF16, 2, FULL, POS, NORM>), grid, blk, 0, st, p); break;
    case 4: hipLaunchKernelGGL((score_gqa_kernel<BF16, 4, FULL, POS, NORM>), grid, blk, 0, st, p); break;
    case 8: hipLaunchKernelGGL((score_gqa_kernel<BF16, 8, FULL, POS, NORM>), grid, blk, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16, bool POS, bool NORM>
hipError_t launch_full(const GqaParams &p, int ppq, dim3 grid, hipStream_t st) {
  const int pieces = p.d * (BF16 ? 2 : 4) / 16;
  return pieces == 4 * ppq ? launch_ppq<BF16, true, POS, NORM>(p, ppq, grid, st)
                           : launch_ppq<BF16, false, POS, NORM>(p, ppq, grid, st);
}

}  // namespace

// Kernel B over the raw scores and chunk sums kernel A wrote.
hipError_t launch_finish(const GqaParams &p, dim3 grid, hipStream_t st) {
  const dim3 blk(kScoreThreads);
  switch (group_bound(p.G)) {
    case 1: hipLaunchKernelGGL(gqa_finish_kernel<1>, grid, blk, 0, st, p); break;
    case 2: hipLaunchKernelGGL(gqa_finish_kernel<2>, grid, blk, 0, st, p); break;
    case 4: hipLaunchKernelGGL(gqa_finish_kernel<4>, grid, blk, 0, st, p); break;
    case 8: hipLaunchKernelGGL(gqa_finish_kernel<8>, grid, blk, 0, st, p); break;
    case 16: hipLaunchKernelGGL(gqa_finish_kernel<16>, grid, blk, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16, bool HALF, int LAYOUT, bool NORM, int GM>
hipError_t launch_gqa_rot_lpk(const GqaParams &p, int lpk, dim3 grid, hipStream_t st) {
  const dim3 blk(kScoreThreads);
  switch (lpk) {
    case 1: hipLaunchKernelGGL((gqa_rotated_kernel<BF16, 1, HALF, LAYOUT, NORM, GM>), grid, blk, 0, st, p); break;
    case 2: hipLaunchKernelGGL((gqa_rotated_kernel<BF16, 2, HALF, LAYOUT, NORM, GM>), grid, blk, 0, st, p); break;
    case 4: hipLaunchKernelGGL((gqa_rotated_kernel<BF16, 4, HALF, LAYOUT, NORM, GM>), grid, blk, 0, st, p); break;
    case 8: hipLaunchKernelGGL((gqa_rotated_kernel<BF16, 8, HALF, LAYOUT, NORM, GM>), grid, blk, 0, st, p); break;
    case 16: hipLaunchKernelGGL((gqa_rotated_kernel<BF16, 16, HALF, LAYOUT, NORM, GM>), grid, blk, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16, bool HALF, int LAYOUT, bool NORM>
hipError_t launch_gqa_rot_group(const GqaParams &p, int lpk, dim3 grid, hipStream_t st) {
  switch (group_bound(p.G)) {
    case 1: return launch_gqa_rot_lpk<BF16, HALF, LAYOUT, NORM, 1>(p, lpk, grid, st);
    case 2: return launch_gqa_rot_lpk<BF16, HALF, LAYOUT, NORM, 2>(p, lpk, grid, st);
    case 4: return launch_gqa_rot_lpk<BF16, HALF, LAYOUT, NORM, 4>(p, lpk, grid, st);
    case 8: return launch_gqa_rot_lpk<BF16, HALF, LAYOUT, NORM, 8>(p, lpk, grid, st);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16, bool HALF, int LAYOUT>
hipError_t launch_gqa_rot_norm(const GqaParams &p, int lpk, dim3 grid, hipStream_t st) {
  return p.qabs ? launch_gqa_rot_group<BF16, HALF, LAYOUT, true>(p, lpk, grid, st)
                : launch_gqa_rot_group<BF16, HALF, LAYOUT, false>(p, lpk, grid, st);
}

template <bool BF16>
hipError_t launch_gqa_rot_layout(const GqaParams &p, int layout, int lpk, dim3 grid, hipStream_t st) {
  if (p.half) {
    switch (layout) {
      case 0: return launch_gqa_rot_norm<BF16, true, 0>(p, lpk, grid, st);
      case 1: return launch_gqa_rot_norm<BF16, true, 1>(p, lpk, grid, st);
      case 2: return launch_gqa_rot_norm<BF16, true, 2>(p, lpk, grid, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (layout) {
    case 0: return launch_gqa_rot_norm<BF16, false, 0>(p, lpk, grid, st);
    case 1: return launch_gqa_rot_norm<BF16, false, 1>(p, lpk, grid, st);
    case 2: return launch_gqa_rot_norm<BF16, false, 2>(p, lpk, grid, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_score_gqa(const GqaParams &p, int dtype_bf16, int pieces_per_lane, hipStream_t st) {
  const long long blocks = static_cast<long long>(p.L) * p.S * p.H * p.chunks_per_head;
  if (blocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(blocks));
  const bool pos = p.pos != nullptr, norm = p.qabs != nullptr;
  const int ppq = pieces_per_lane;
  hipError_t e;
  // bf16 rows of 4, 8 or 16 pieces (head_dim 32, 64, 128), G <= 4, contiguous positions, rows
  // addressable with 32-bit offsets: the VALU stream form; everything else: the matrix cores
  const int pieces = p.d * (dtype_bf16 ? 2 : 4) / 16;
  const bool stream = dtype_bf16 && !pos && p.G <= KV_GQA_STREAM_MAX_G && (pieces == 4 || pieces == 8 || pieces == 16) &&
                      static_cast<long long>(p.t_cap + 2 * kGqaChunk) * p.d * 2 < (1ll << 31);
  if (stream)
    e = norm ? launch_stream<true>(p, pieces, grid, st) : launch_stream<false>(p, pieces, grid, st);
  else if (dtype_bf16)
    e = pos ? (norm ? launch_full<true, true, true>(p, ppq, grid, st) : launch_full<true, true, false>(p, ppq, grid, st))
            : (norm ? launch_full<true, false, true>(p, ppq, grid, st) : launch_full<true, false, false>(p, ppq, grid, st));
  else
    e = pos ? (norm ? launch_full<false, true, true>(p, ppq, grid, st) : launch_full<false, true, false>(p, ppq, grid, st))
            : (norm ? launch_full<false, false, true>(p, ppq, grid, st) : launch_full<false, false, false>(p, ppq, grid, st));
  if (e != hipSuccess) return e;
  return launch_finish(p, grid, st);
}

hipError_t launch_score_gqa_rotated(const GqaParams &p, int dtype_bf16, int layout, int lanes_per_key,
                                    hipStream_t st) {
  const long long blocks = static_cast<long long>(p.L) * p.S * p.H * p.chunks_per_head;
  if (blocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(blocks));
  const hipError_t e = dtype_bf16 ? launch_gqa_rot_layout<true>(p, layout, lanes_per_key, grid, st)
                                  : launch_gqa_rot_layout<false>(p, layout, lanes_per_key, grid, st);
  if (e != hipSuccess) return e;
  return launch_finish(p, grid, st);
}

}  // namespace kvevict

// Grouped-query scores: per-query-head scores, z-normalised per query head, max over the group.
//
// What is computed: "TriAttention: Efficient Long Reasoning with Trigonometric
// KV Compression" (structured summary 3.4, "KV Cache Pruning Procedure", the
// GQA handling): each of the G query heads sharing a KV head scores every
// cached key with its own centre, its scores are normalised to zero mean and
// unit (population) standard deviation over the head's T cached keys, and the
// key's final score is the maximum of its G normalised scores.
//
// Kernel A reads every key once. Per band it forms y_f = exp(i omega_f m) *
// conj(k_f) once (m = t - p, the phase carried by the same recurrence as the
// single-centre kernel, or derived exactly per key for explicit positions),
// then each query head costs two FMAs: Re(u_{g,f} y_f). It writes the G raw
// scores and, per (head, chunk of keys), fp64 sums of s and s^2 for each g.
// Kernel B reduces a head's chunk sums in a fixed order (deterministic, no
// atomics) and writes max_g (s_g - mu_g) / sigma_g (0 for a query head whose
// scores do not vary).
#include "kv_internal.hpp"

namespace kvevict {
namespace {

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

__device__ __forceinline__ float2 cis_rev(double rev, double m) {
  const double x = rev * m;
  const double r = x - rint(x);
  float sn, cs;
  sincospif(2.0f * static_cast<float>(r), &sn, &cs);
  return make_float2(cs, sn);
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

// GM: group size rounded up to a power of two; query heads g >= p.G have zero centres and are not stored.
template <bool BF16, int LPK, bool POS, bool NORM, int GM>
__global__ __launch_bounds__(kScoreThreads) void score_gqa_kernel(const GqaParams p) {
  constexpr int BPL = BF16 ? 4 : 2;
  constexpr int KPS = 64 / LPK;
  constexpr int STEPS = LPK;
  constexpr int SUB = STEPS < 8 ? STEPS : 8;
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int NW = kScoreThreads / 64;
  __shared__ double part[NW][GM][2];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int gl = lane % LPK;  // band group of this lane
  const int kk = lane / LPK;
  const int head = blockIdx.x / p.chunks_per_head;
  const int chunk = blockIdx.x - head * p.chunks_per_head;
  const int h = head % p.H;
  const int s = (head / p.H) % p.S;
  const int l = head / (p.H * p.S);

  const int T = min(max(p.seq_len[s], 0), p.t_cap);
  const int wave_first = chunk * kScoreChunk + wave * (kScoreBatchesPerWave * 64);
  const double tq = static_cast<double>(p.t_cur[s]);

  const bool live = gl * BPL < p.F;
  float2 u[GM][BPL], w[BPL], z[BPL];
  float cn[GM][BPL];
  double rev[BPL];
  const size_t lhg = (static_cast<size_t>(l) * p.H + h) * p.G;
#pragma unroll
  for (int i = 0; i < BPL; ++i) {
    const int b = gl * BPL + i;
    rev[i] = live ? p.rev[b] : 0.0;
    w[i] = live ? cis_rev(rev[i], -static_cast<double>(KPS)) : make_float2(1.f, 0.f);
#pragma unroll
    for (int g = 0; g < GM; ++g) {
      if (live && g < p.G) {
        const float2 q = reinterpret_cast<const float2 *>(p.qbar + (lhg + g) * p.d)[b];
        u[g][i] = cmul(q, p.A[b]);
        float c = 0.f;
        if (NORM) {
          const float qa = p.qabs[(lhg + g) * p.F + b];
          c = qa > 0.f ? qa - __builtin_amdgcn_sqrtf(fmaf(q.x, q.x, q.y * q.y)) : 0.f;
        }
        cn[g][i] = c;
      } else {
        u[g][i] = make_float2(0.f, 0.f);
        cn[g][i] = 0.f;
      }
    }
  }
  double sum[GM], sum2[GM];
#pragma unroll
  for (int g = 0; g < GM; ++g) sum[g] = sum2[g] = 0.0;

  const size_t slot0 = static_cast<size_t>(head) * p.t_cap;
  const size_t row_bytes = static_cast<size_t>(p.d) * EB;
  const char *Kh = static_cast<const char *>(p.K) + slot0 * row_bytes + static_cast<size_t>(live ? gl : 0) * 16;
  if (!POS && wave_first < T) {
    const double m0 = tq - static_cast<double>(wave_first + kk);
#pragma unroll
    for (int i = 0; i < BPL; ++i) z[i] = cis_rev(rev[i], m0);
  }
#pragma unroll 1
  for (int nb = 0; nb < kScoreBatchesPerWave; ++nb) {
    const int j0 = wave_first + nb * 64;
    if (j0 >= T) break;
    float acc[GM][STEPS];
#pragma unroll
    for (int st0 = 0; st0 < STEPS; st0 += SUB) {
      uint4 data[SUB];
      int32_t pj[SUB];
#pragma unroll
      for (int t = 0; t < SUB; ++t) {
        const int j = j0 + (st0 + t) * KPS + kk;
        const int jc = j < T ? j : 0;  // slots past T read row 0; their sums are not used
        const v4u32 v = __builtin_nontemporal_load(reinterpret_cast<const v4u32 *>(Kh + jc * row_bytes));
        data[t] = make_uint4(v[0], v[1], v[2], v[3]);
        if (POS) pj[t] = p.pos[slot0 + jc];
      }
#pragma unroll
      for (int t = 0; t < SUB; ++t) {
        if (POS) {
          const double m = tq - static_cast<double>(pj[t]);
#pragma unroll
          for (int i = 0; i < BPL; ++i) z[i] = cis_rev(rev[i], m);
        }
        const uint32_t wd[4] = {data[t].x, data[t].y, data[t].z, data[t].w};
        float a[GM];
#pragma unroll
        for (int g = 0; g < GM; ++g) a[g] = 0.f;
#pragma unroll
        for (int i = 0; i < BPL; ++i) {
          const float re = BF16 ? __uint_as_float(wd[i] << 16) : __uint_as_float(wd[2 * i]);
          const float im = BF16 ? __uint_as_float(wd[i] & 0xffff0000u) : __uint_as_float(wd[2 * i + 1]);
          // y = z * conj(k): shared by every query head of the group
          const float yx = fmaf(z[i].x, re, z[i].y * im);
          const float yy = fmaf(z[i].y, re, -z[i].x * im);
          const float kabs = NORM ? __builtin_amdgcn_sqrtf(fmaf(re, re, im * im)) : 0.f;
#pragma unroll
          for (int g = 0; g < GM; ++g) {
            a[g] = fmaf(u[g][i].x, yx, a[g]);
            a[g] = fmaf(-u[g][i].y, yy, a[g]);
            if (NORM) a[g] = fmaf(cn[g][i], kabs, a[g]);
          }
        }
#pragma unroll
        for (int g = 0; g < GM; ++g) acc[g][st0 + t] = live ? a[g] : 0.f;
        if (!POS) {
#pragma unroll
          for (int i = 0; i < BPL; ++i) z[i] = cmul(z[i], w[i]);
        }
      }
    }
    const int jj = j0 + gl * KPS + kk;
#pragma unroll
    for (int g = 0; g < GM; ++g) {
      const float sc = reduce_scatter<STEPS>(acc[g], gl);
      if (jj < T && g < p.G) {
        __builtin_nontemporal_store(sc, p.raw + (static_cast<size_t>(head) * p.G + g) * p.t_cap + jj);
        sum[g] += static_cast<double>(sc);
        sum2[g] += static_cast<double>(sc) * static_cast<double>(sc);
      }
    }
  }
  // per (head, chunk) sums of s and s^2 for each query head, in a fixed reduction order
#pragma unroll
  for (int g = 0; g < GM; ++g) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      sum[g] += __shfl_xor(sum[g], off, 64);
      sum2[g] += __shfl_xor(sum2[g], off, 64);
    }
    if (lane == 0) {
      part[wave][g][0] = sum[g];
      part[wave][g][1] = sum2[g];
    }
  }
  __syncthreads();
  if (static_cast<int>(threadIdx.x) < p.G) {
    const int g = threadIdx.x;
    double a = 0.0, b = 0.0;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) {
      a += part[wv][g][0];
      b += part[wv][g][1];
    }
    double *dst = p.partials + ((static_cast<size_t>(head) * p.chunks_per_head + chunk) * p.G + g) * 2;
    dst[0] = a;
    dst[1] = b;
  }
}

// One workgroup per (head, chunk): reduce the head's chunk sums, then normalise and take the max.
template <int GM>
__global__ __launch_bounds__(kScoreThreads) void gqa_finish_kernel(const GqaParams p) {
  __shared__ double stats[GM][2];  // mean, 1/std (0 when the std is 0)
  const int head = blockIdx.x / p.chunks_per_head;
  const int chunk = blockIdx.x - head * p.chunks_per_head;
  const int s = (head / p.H) % p.S;
  const int T = min(max(p.seq_len[s], 0), p.t_cap);
  const int j0 = chunk * kScoreChunk;
  if (j0 >= T) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave == 0) {
    const int n_chunks = (T + kScoreChunk - 1) / kScoreChunk;
#pragma unroll
    for (int g = 0; g < GM; ++g) {
      if (g >= p.G) break;
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
  }
  __syncthreads();
  const int jend = min(j0 + kScoreChunk, T);
  for (int j = j0 + static_cast<int>(threadIdx.x); j < jend; j += kScoreThreads) {
    double best = -INFINITY;
#pragma unroll
    for (int g = 0; g < GM; ++g) {
      if (g >= p.G) break;
      const double sc = p.raw[(static_cast<size_t>(head) * p.G + g) * p.t_cap + j];
      best = fmax(best, (sc - stats[g][0]) * stats[g][1]);
    }
    p.scores[static_cast<size_t>(head) * p.t_cap + j] = static_cast<float>(best);
  }
}

int group_bound(int G) {
  int gm = 1;
  while (gm < G) gm <<= 1;
  return gm;
}

template <bool BF16, int LPK, bool POS, bool NORM>
hipError_t launch_g(const GqaParams &p, dim3 grid, hipStream_t st) {
  const dim3 blk(kScoreThreads);
  const int gm = group_bound(p.G);
  switch (gm) {
    case 1: hipLaunchKernelGGL((score_gqa_kernel<BF16, LPK, POS, NORM, 1>), grid, blk, 0, st, p); break;
    case 2: hipLaunchKernelGGL((score_gqa_kernel<BF16, LPK, POS, NORM, 2>), grid, blk, 0, st, p); break;
    case 4: hipLaunchKernelGGL((score_gqa_kernel<BF16, LPK, POS, NORM, 4>), grid, blk, 0, st, p); break;
    case 8: hipLaunchKernelGGL((score_gqa_kernel<BF16, LPK, POS, NORM, 8>), grid, blk, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16, bool POS, bool NORM>
hipError_t launch_lpk_g(const GqaParams &p, int lpk, dim3 grid, hipStream_t st) {
  switch (lpk) {
    case 1: return launch_g<BF16, 1, POS, NORM>(p, grid, st);
    case 2: return launch_g<BF16, 2, POS, NORM>(p, grid, st);
    case 4: return launch_g<BF16, 4, POS, NORM>(p, grid, st);
    case 8: return launch_g<BF16, 8, POS, NORM>(p, grid, st);
    case 16: return launch_g<BF16, 16, POS, NORM>(p, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_score_gqa(const GqaParams &p, int dtype_bf16, int lanes_per_key, hipStream_t st) {
  const long long blocks = static_cast<long long>(p.L) * p.S * p.H * p.chunks_per_head;
  if (blocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(blocks));
  const bool pos = p.pos != nullptr, norm = p.qabs != nullptr;
  hipError_t e;
  if (dtype_bf16)
    e = pos ? (norm ? launch_lpk_g<true, true, true>(p, lanes_per_key, grid, st)
                    : launch_lpk_g<true, true, false>(p, lanes_per_key, grid, st))
            : (norm ? launch_lpk_g<true, false, true>(p, lanes_per_key, grid, st)
                    : launch_lpk_g<true, false, false>(p, lanes_per_key, grid, st));
  else
    e = pos ? (norm ? launch_lpk_g<false, true, true>(p, lanes_per_key, grid, st)
                    : launch_lpk_g<false, true, false>(p, lanes_per_key, grid, st))
            : (norm ? launch_lpk_g<false, false, true>(p, lanes_per_key, grid, st)
                    : launch_lpk_g<false, false, false>(p, lanes_per_key, grid, st));
  if (e != hipSuccess) return e;
  const dim3 blk(kScoreThreads);
  switch (group_bound(p.G)) {
    case 1: hipLaunchKernelGGL(gqa_finish_kernel<1>, grid, blk, 0, st, p); break;
    case 2: hipLaunchKernelGGL(gqa_finish_kernel<2>, grid, blk, 0, st, p); break;
    case 4: hipLaunchKernelGGL(gqa_finish_kernel<4>, grid, blk, 0, st, p); break;
    case 8: hipLaunchKernelGGL(gqa_finish_kernel<8>, grid, blk, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvevict

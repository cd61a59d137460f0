// Per-head exact top-n selection with pinned prompt and recent window, for gfx950.
//
// What is computed: "TriAttention: Efficient Long Reasoning with
// Trigonometric KV Compression" (structured summary, section 3.4, "KV Cache
// Pruning Procedure": keep the top B when the cache exceeds B), "Random
// Attention: Rethinking KV Cache Eviction for Efficient Reasoning" (section
// 2: a recent buffer that is never scored, top-K of the candidates, Eq. 2;
// section 3: the prompt is never evicted, and each candidate gets an i.i.d.
// uniform score drawn per KV head at every eviction, Eq. 3 / Algorithm 1;
// Appendix F: keep-sets sorted chronologically) and "TriAttention" (blog
// walkthrough, eviction step: union-based selection over per-head top-k sets).
//
// One workgroup owns one (layer, seq, KV head). Its T slot keys live in
// registers; thread t holds, for each round i, the four consecutive slots
// 4*(i*NT + t) .. +3, so every round is one fully coalesced 16-byte-per-lane
// load and the head's scores are read from HBM exactly once:
//  1. Keys: fp32 scores mapped to order-preserving uint32 (NaN -> -inf,
//     -0 -> +0) or, for the random selector, word 0 of Philox4x32-10.
//  2. A 1024-bin LDS histogram (scores binned by value between the smallest
//     and largest finite candidate, random keys by their top 10 bits) finds
//     the bin holding the n_sel-th largest key; every key in a higher bin is
//     larger.
//  3. That bin's keys, usually a few dozen, are listed in LDS and ranked
//     directly to give the n_sel-th largest key thr and how many keys equal to
//     thr must be taken (need). A crowded bin instead goes through 8-bit radix
//     passes over a 256-bin histogram, from the highest bit where its keys
//     differ (an OR/AND block reduction).
//  4. One ordered scan in slot order counts, before each slot, the slots kept
//     unconditionally (pinned, or above thr) and the slots equal to thr. A
//     kept slot's output index is then (unconditional before) +
//     min(equal before, need): ties go to the lower slot and the kept list is
//     written in ascending order without a sort.
#include "kv_internal.hpp"

#ifndef KV_SELECT_WIDE
#define KV_SELECT_WIDE 0
#endif
// Top-k and random (union) caches longer than this run the kernel that re-reads its keys. Past
// 32768 slots the 1024 x 64 register tier spills; the re-reading kernel was measured faster there
// for top-k (40000 slots: 0.32 -> 0.22 ms; 65536: within 4 %) and random (0.48 -> 0.35, 0.66 ->
// 0.57 ms), slower for the union (1.34 -> 1.54, 1.64 -> 2.72 ms), on 1152 heads.
#ifndef KV_SELECT_STREAM_ABOVE
#define KV_SELECT_STREAM_ABOVE 32768
#endif
#ifndef KV_UNION_STREAM_ABOVE
#define KV_UNION_STREAM_ABOVE 65536
#endif

namespace kvevict {
namespace {

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11): 10 rounds of two 32x32->64 products on counter
// words 0 and 2 with the published multipliers, the key advanced between
// rounds by the published Weyl constants. Returns output word 0.
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
  constexpr uint32_t kMulA = 0xD2511F53u, kMulB = 0xCD9E8D57u;
  constexpr uint32_t kWeylA = 0x9E3779B9u, kWeylB = 0xBB67AE85u;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    // one 32 x 32 -> 64-bit product per multiplier (v_mad_u64_u32) gives both halves
    const uint64_t pa = static_cast<uint64_t>(kMulA) * c0, pb = static_cast<uint64_t>(kMulB) * c2;
    const uint32_t lo_a = static_cast<uint32_t>(pa), hi_a = static_cast<uint32_t>(pa >> 32);
    const uint32_t lo_b = static_cast<uint32_t>(pb), hi_b = static_cast<uint32_t>(pb >> 32);
    const uint32_t n0 = hi_b ^ c1 ^ k0;
    const uint32_t n2 = hi_a ^ c3 ^ k1;
    c0 = n0;
    c1 = lo_b;
    c2 = n2;
    c3 = lo_a;
    k0 += kWeylA;
    k1 += kWeylB;
  }
  return c0;
}

// Order-preserving uint32 image of an fp32 score: NaN ranks as -inf, -0 equals +0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (f != f) b = 0xFF800000u;        // NaN -> -inf
  if ((b << 1) == 0u) b = 0u;         // -0 -> +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inclusive prefix sum across the 64 lanes of a wave with DPP lane moves (no LDS): row
// shifts by 1, 2, 4, 8 scan each row of 16 lanes (bound_ctrl feeds 0 past the row start),
// then the last lane of row 0 is broadcast into row 1 and row 2's into row 3, and the last
// lane of rows 0-1 into rows 2-3. Lanes a move does not write keep the 0 passed as `old`.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x111, 0xf, 0xf, true));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x112, 0xf, 0xf, true));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x114, 0xf, 0xf, true));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x118, 0xf, 0xf, true));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x142, 0xa, 0xf, false));
  x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x143, 0xc, 0xf, false));
  return x;
}

__device__ __forceinline__ uint32_t wave_total(uint32_t incl) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), 63));
}

constexpr uint32_t kKeyNegInf = 0x007FFFFFu;  // order_key(-inf)
constexpr uint32_t kKeyPosInf = 0xFF800000u;  // order_key(+inf)
constexpr int kValueBins = 1024;

// The fp32 value an order key stands for (inverse of order_key on non-NaN values).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Monotone (non-decreasing) map of a key to one of kValueBins bins spanning [fmin, fmax];
// -inf and +inf go to the end bins. Rounded operations that cannot be contracted keep the
// two evaluations of a key (histogram and membership) bit-identical.
__device__ __forceinline__ uint32_t value_bin(uint32_t k, float fmin, float scale) {
  if (k <= kKeyNegInf) return 0u;
  if (k >= kKeyPosInf) return kValueBins - 1u;
  const float x = __fmul_rn(__fsub_rn(key_value(k), fmin), scale);
  return min(static_cast<uint32_t>(x), static_cast<uint32_t>(kValueBins - 1));
}

// value_bin never decreases as the key grows (over all 2^32 keys), so the keys of one bin form an
// interval. Run by one wave: the smallest key whose bin is at least `target`, or 2^32 when none
// is, by a 64-way search over the key space (at most seven rounds). It evaluates the same
// rounded expression as the histogram pass, so the interval test that replaces a second
// evaluation per key agrees with it key for key.
__device__ __forceinline__ uint64_t first_key_reaching(uint32_t target, float fmin, float scale, int lane) {
  uint64_t lo = 0, hi = uint64_t{1} << 32;   // keys below lo stay under target; hi reaches it (2^32: none)
  while (lo < hi) {
    const uint64_t step = (hi - lo + 63) >> 6;
    const uint64_t c = lo + static_cast<uint64_t>(lane) * step;
    const bool reach = c >= hi || value_bin(static_cast<uint32_t>(c), fmin, scale) >= target;
    const uint64_t m = __ballot(reach);
    if (m & 1ull) return lo;
    const int f = m ? __builtin_ctzll(m) : 64;               // first probe that reaches (64: none)
    const uint64_t below = lo + static_cast<uint64_t>(f - 1) * step;  // the last probe that does not
    if (f < 64) hi = min(hi, lo + static_cast<uint64_t>(f) * step);
    lo = below + 1;
  }
  return hi;
}

// Interval [lo, hi] of the keys of bin b, in LDS slots kb[0], kb[1]: scores (value bins) by waves 0
// and 1 of the workgroup (the caller then synchronises), random keys (top 10 bits) directly.
template <bool RANDOM>
__device__ __forceinline__ void bin_interval(uint32_t b, float fmin, float scale, int wave, int lane,
                                             uint32_t *kb) {
  if (RANDOM) {
    if (wave == 0 && lane == 0) {
      kb[0] = b << 22;
      kb[1] = (b << 22) | 0x3FFFFFu;
    }
  } else if (wave < 2) {
    const uint64_t k = first_key_reaching(b + static_cast<uint32_t>(wave), fmin, scale, lane);
    if (lane == 0) kb[wave] = static_cast<uint32_t>(k - static_cast<uint64_t>(wave));  // bin b+1's first, minus one
  }
}

// Run by one wave: lane L owns bins (NBINS/64)*L ...; finds the bin b holding the remaining-th
// largest key (counting from the top) and the number of keys in bins above it.
template <int NBINS>
__device__ __forceinline__ void find_bin(const uint32_t *hist, uint32_t remaining, int lane, uint32_t *found) {
  constexpr int PER = NBINS / 64;
  uint32_t c[PER];
  uint32_t local = 0u;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    c[q] = hist[PER * lane + q];
    local += c[q];
  }
  const uint32_t incl = wave_inclusive_sum(local);
  uint32_t cum = wave_total(incl) - incl;  // keys in bins owned by higher lanes
#pragma unroll
  for (int q = PER - 1; q >= 0; --q) {
    const uint32_t above = cum;
    cum += c[q];
    if (above < remaining && cum >= remaining) {
      found[0] = static_cast<uint32_t>(PER * lane + q);
      found[1] = above;
    }
  }
}

template <int NT>
__device__ __forceinline__ void block_min_max(uint32_t &mn, uint32_t &mx, uint32_t *lds /* 2*NT/64 */) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mn = min(mn, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mn), off, 64)));
    mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), off, 64)));
  }
  if (lane == 0) {
    lds[wave] = mn;
    lds[NW + wave] = mx;
  }
  __syncthreads();
  mn = 0xFFFFFFFFu;
  mx = 0u;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    mn = min(mn, lds[i]);
    mx = max(mx, lds[NW + i]);
  }
  __syncthreads();  // lds may be reused right after
}

template <int NT>
__device__ __forceinline__ void block_or_and(uint32_t &o, uint32_t &a, uint32_t *lds /* 2*NT/64 */) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    o |= __shfl_xor(o, off, 64);
    a &= __shfl_xor(a, off, 64);
  }
  if (lane == 0) {
    lds[wave] = o;
    lds[NW + wave] = a;
  }
  __syncthreads();
  o = 0u;
  a = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    o |= lds[i];
    a &= lds[NW + i];
  }
  __syncthreads();  // lds may be reused right after
}

// In-place exclusive scan of n values held in LDS, run by one wave (n may exceed 64).
__device__ __forceinline__ void wave_exclusive_scan_lds(uint32_t *a, int n, int lane) {
  uint32_t carry = 0u;
  for (int c = 0; c < n; c += 64) {
    const uint32_t v = (c + lane < n) ? a[c + lane] : 0u;
    const uint32_t x = wave_inclusive_sum(v);
    if (c + lane < n) a[c + lane] = carry + x - v;
    carry += wave_total(x);
  }
}

// Threshold among a short member list held in LDS (list[0..m), zero-padded to a multiple of 4;
// keys are >= 0, so a pad only ever ties with a key equal to 0): the key with fewer than
// `remaining` larger members and at least `remaining` larger-or-equal ones, how many keys equal
// to it are taken, and how many there are. Every thread that finds it writes the same triple into
// found[0..2].
template <int NT>
__device__ __forceinline__ void rank_members(const uint32_t *list, uint32_t m, uint32_t remaining,
                                             uint32_t *found) {
  const uint32_t m4 = (m + 3u) & ~3u, pads = m4 - m;
  for (uint32_t t = threadIdx.x; t < m; t += NT) {
    const uint32_t k = list[t];
    uint32_t gt = 0u, ge = 0u;
    for (uint32_t u = 0; u < m4; u += 4) {
      const uint4 v = *reinterpret_cast<const uint4 *>(list + u);
      gt += (v.x > k) + (v.y > k) + (v.z > k) + (v.w > k);
      ge += (v.x >= k) + (v.y >= k) + (v.z >= k) + (v.w >= k);
    }
    if (k == 0u) ge -= pads;
    if (gt < remaining && ge >= remaining) {
      found[0] = k;
      found[1] = remaining - gt;
      found[2] = ge - gt;
    }
  }
}

// Largest member list ranked directly (it lives in the value histogram's LDS with 4 slots of
// padding to spare); longer lists go through the radix passes.
template <int NT>
constexpr uint32_t member_cap() { return 2 * NT < kValueBins - 4 ? 2 * NT : kValueBins - 4; }

// The three rankings share one kernel body. KIND 0 (top-k): keys are the fp32 scores. KIND 1
// (random): keys are Philox words. KIND 2 (union, "TriAttention" blog, eviction step): G + 1
// passes over the same registers -- pass g < G ranks the evictable slots by query head g's own
// score and adds its top-k to a per-thread union bit mask; the last pass ranks by the combined
// score, inside the union when it holds at least n_sel slots, otherwise over the rest of the
// evictable range with the whole union kept. Every pass is a threshold search (steps 2-3) and an
// ordered scan (step 4); top-k and random run exactly one pass.
//
// VEC (score keys only): every score row is 16-byte aligned and t_cap is a multiple of 4, so
// each round is one float4 load per lane (slots past T are loaded but never used).
template <int NT, int KPT, int KIND, bool VEC>
__global__ __launch_bounds__(NT) void select_kernel(const SelectParams p) {
  constexpr int NW = NT / 64;
  constexpr int R = KPT / 4;   // rounds of four consecutive slots per thread
  constexpr bool RANDOM = KIND == 1, UNION = KIND == 2;
  __shared__ __align__(16) uint32_t hist[kValueBins];
  __shared__ uint32_t red[2 * NW];
  __shared__ uint32_t tot_a[R * NW];   // per (round, wave): slots kept unconditionally
  __shared__ uint32_t tot_e[R * NW];   // per (round, wave): slots whose key equals thr
  __shared__ uint32_t found[3];
  __shared__ uint32_t n_members;
  __shared__ uint32_t kb[2];   // key interval of the threshold's bin

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int head = blockIdx.x;
  const int h = head % p.H;
  const int s = (head / p.H) % p.S;
  const int l = head / (p.H * p.S);

  const int T = min(max(p.seq_len[s], 0), p.t_cap);
  const int P = min(max(p.prompt_len[s], 0), min(p.prompt_cap, T));
  const int B = p.budget;
  int32_t *out = p.kept + static_cast<size_t>(head) * p.b_cap;
  const bool writer = (l == 0 && h == 0 && tid == 0);

  if (T <= B) {  // nothing to compress: keep 0..T-1
    for (int r = tid; r < p.b_cap; r += NT) out[r] = r < T ? r : -1;
    if (writer) p.n_kept[s] = T;
    return;
  }
  const int Rw = min(p.recent, min(max(0, B - P), T - P));
  const int e_lo = P, e_hi = T - Rw;
  const int n_sel = max(0, B - P - Rw);
  const int n_kept = max(B, P);
  const int n_cand = e_hi - e_lo;

  auto slot_of = [&](int i) { return 4 * ((i >> 2) * NT + tid) + (i & 3); };
  uint64_t cand = 0ull;  // bit i: key[i] is an evictable candidate
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int j = slot_of(i);
    cand |= static_cast<uint64_t>(j >= e_lo && j < e_hi) << i;
  }
  const size_t slot0 = static_cast<size_t>(head) * p.t_cap;
  const int passes = UNION ? (n_sel > 0 ? p.G : 0) + 1 : 1;
  const int k_head = UNION ? (p.k_per_head > 0 ? p.k_per_head : (n_sel + p.G - 1) / p.G) : 0;
  uint64_t umask = 0ull;    // union: slots some query head ranks in its top-k

  uint32_t key[KPT];
#pragma unroll 1
  for (int pass = 0; pass < passes; ++pass) {
    const bool last = pass == passes - 1;
    // ---- 1. keys: key[4*i + q] belongs to slot 4*(i*NT + tid) + q
    if (!RANDOM) {
      const float *row = p.scores + slot0;
      if (UNION && !last) row = p.head_scores + (static_cast<size_t>(head) * p.G + pass) * p.t_cap;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int j4 = 4 * (i * NT + tid);
        if (VEC) {
          float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
          if (j4 < p.t_cap) f = *reinterpret_cast<const float4 *>(row + j4);
          key[4 * i] = order_key(f.x);
          key[4 * i + 1] = order_key(f.y);
          key[4 * i + 2] = order_key(f.z);
          key[4 * i + 3] = order_key(f.w);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) key[4 * i + q] = (j4 + q < T) ? order_key(row[j4 + q]) : 0u;
        }
      }
    } else {
      const uint32_t c1 = p.shared_draw ? 0u : (static_cast<uint32_t>(l) << 16) | static_cast<uint32_t>(h);
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const int j = slot_of(i);
        uint32_t k = 0u;
        if (j >= e_lo && j < e_hi) {
          const uint32_t c0 = p.pos ? static_cast<uint32_t>(p.pos[slot0 + j]) : static_cast<uint32_t>(j);
          k = philox_word0(c0, c1, static_cast<uint32_t>(s), p.event, p.seed_lo, p.seed_hi);
        }
        key[i] = k;
      }
    }
    // Union, last pass: rank by the combined score with the union folded into the keys. A long
    // union (>= n_sel slots) drops every other slot to key 0, below any score; a short one lifts
    // its own slots to the top key, above any score, so the top-up comes from the rest.
    int p_sel = n_sel;
    if (UNION && !last) {
      p_sel = k_head;
    } else if (UNION) {
      uint32_t nu = static_cast<uint32_t>(__popcll(umask));
      nu = wave_total(wave_inclusive_sum(nu));
      if (lane == 0) red[wave] = nu;
      __syncthreads();
      int n_union = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) n_union += static_cast<int>(red[w]);
      __syncthreads();
      const bool long_union = n_union >= n_sel;
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const bool in_u = (umask >> i) & 1ull;
        if (long_union && !in_u) key[i] = 0u;
        if (!long_union && in_u) key[i] = 0xFFFFFFFFu;
      }
    }

    // ---- 2./3. threshold: thr = p_sel-th largest candidate key; take `need` of the keys == thr
    // mode: 0 = select none, 1 = select all candidates, 2 = threshold rule
    int mode;
    uint32_t thr = 0u, need = 0u;
    bool all_ties = false;  // every key equal to thr is taken
    if (p_sel <= 0 || n_cand <= 0) {
      mode = 0;
    } else if (p_sel >= n_cand) {
      mode = 1;
    } else {
      mode = 2;
      uint32_t remaining = static_cast<uint32_t>(p_sel);
      uint64_t mem = cand;  // keys the exact radix passes still have to order
      bool ranked = false;  // threshold found by ranking a short member list
      // Pass 1: 1024 bins. Scores are binned uniformly in value between the smallest and largest
      // finite candidate (binning by value keeps a concentrated score distribution from piling
      // into a few bins); uniform random keys by their top 10 bits. The binning is monotone, so
      // the threshold lies in one bin and every key in a higher bin is strictly larger; the exact
      // step then only sees that bin's keys.
      bool binned = RANDOM;
      float fmin = 0.f, scale = 0.f;
      if (!RANDOM) {
        uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
          if (((cand >> i) & 1ull) && key[i] > kKeyNegInf && key[i] < kKeyPosInf) {
            kmn = min(kmn, key[i]);
            kmx = max(kmx, key[i]);
          }
        }
        block_min_max<NT>(kmn, kmx, red);
        fmin = key_value(kmn);
        const float fmax = key_value(kmx);
        scale = static_cast<float>(kValueBins) / (fmax - fmin);
        binned = kmn < kmx && scale > 0.f && scale < 3.0e38f;
      }
      {
        auto bin_of = [&](uint32_t k) { return RANDOM ? (k >> 22) : value_bin(k, fmin, scale); };
        if (binned) {
          for (int i = tid; i < kValueBins; i += NT) hist[i] = 0u;
          if (tid == 0) n_members = 0u;
          __syncthreads();
#pragma unroll
          for (int i = 0; i < KPT; ++i)
            if ((cand >> i) & 1ull) atomicAdd(&hist[bin_of(key[i])], 1u);
          __syncthreads();
          if (wave == 0) find_bin<kValueBins>(hist, remaining, lane, found);
          __syncthreads();
          const uint32_t b = found[0];
          remaining -= found[1];
          mem = 0ull;
          // Membership in the threshold's bin. With 32 or more keys per thread, testing each key
          // against the bin's key interval (found once by waves 0 and 1) beats evaluating its bin
          // again; with fewer, the search and its barrier cost more than they save (2176-slot
          // heads: 0.095 -> 0.111 ms). A random key's bin is a shift, cheaper than either.
          if constexpr (!RANDOM && KPT >= 32) {
            bin_interval<RANDOM>(b, fmin, scale, wave, lane, kb);
            __syncthreads();
            const uint32_t klo = kb[0], khi = kb[1];
#pragma unroll
            for (int i = 0; i < KPT; ++i)
              if (((cand >> i) & 1ull) && key[i] >= klo && key[i] <= khi) mem |= 1ull << i;
          } else {
#pragma unroll
            for (int i = 0; i < KPT; ++i)
              if (((cand >> i) & 1ull) && bin_of(key[i]) == b) mem |= 1ull << i;
          }
          __syncthreads();  // `found` and `hist` are reused below
          // The threshold's bin usually holds a few keys: list them in LDS (hist is free) and rank
          // them directly instead of running the radix passes.
#pragma unroll
          for (int i = 0; i < KPT; ++i) {
            if ((mem >> i) & 1ull) {
              const uint32_t at = atomicAdd(&n_members, 1u);
              if (at < member_cap<NT>()) hist[at] = key[i];
            }
          }
          __syncthreads();
          const uint32_t m = n_members;
          if (m <= member_cap<NT>()) {
            if (tid < 4) hist[m + tid] = 0u;   // pad to a multiple of 4 (m + 3 < kValueBins)
            __syncthreads();
            rank_members<NT>(hist, m, remaining, found);
            __syncthreads();
            thr = found[0];
            need = found[1];
            all_ties = found[2] == need;   // equal keys share the threshold's bin: all are listed
            ranked = true;
          }
          __syncthreads();  // `found`, `hist` and n_members are reused below
        }
      }
      // Exact radix passes over the member keys, from their highest differing bit.
      if (!ranked) {
        uint32_t kor = 0u, kand = 0xFFFFFFFFu;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
          if ((mem >> i) & 1ull) {
            kor |= key[i];
            kand &= key[i];
          }
        }
        block_or_and<NT>(kor, kand, red);
        const uint32_t diff = kor ^ kand;
        if (diff == 0u) {
          thr = kand;  // all member keys equal
        } else {
          const int top = 31 - __clz(diff);
          uint32_t mask = top == 31 ? 0u : ~((2u << top) - 1u);
          uint32_t prefix = kand & mask;
          for (int hi = top; hi >= 0;) {
            const int lo = hi >= 7 ? hi - 7 : 0;
            const uint32_t dmask = (1u << (hi - lo + 1)) - 1u;
            for (int i = tid; i < 256; i += NT) hist[i] = 0u;
            __syncthreads();
#pragma unroll
            for (int i = 0; i < KPT; ++i) {
              if (((mem >> i) & 1ull) && (key[i] & mask) == prefix) atomicAdd(&hist[(key[i] >> lo) & dmask], 1u);
            }
            __syncthreads();
            if (wave == 0) find_bin<256>(hist, remaining, lane, found);
            __syncthreads();
            const uint32_t digit = found[0];
            remaining -= found[1];
            prefix |= digit << lo;
            mask |= dmask << lo;
            hi = lo - 1;
            __syncthreads();  // everyone has read `found` before the next pass may overwrite it
          }
          thr = prefix;
        }
        need = remaining;
      }
    }

    // ---- 4. one ordered scan: unconditional (A) and equal-to-thr (E) slots before each slot.
    // The last pass writes the kept list; a union head pass adds its top-k to the union.
    uint64_t fa = 0ull, fe = 0ull;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const bool c = (cand >> i) & 1ull;
      const bool pinned = last && !c && slot_of(i) < T;  // prompt or recent window
      const bool a = pinned || (c && (mode == 1 || (mode == 2 && key[i] > thr)));
      const bool e = c && mode == 2 && key[i] == thr;
      fa |= static_cast<uint64_t>(a) << i;
      fe |= static_cast<uint64_t>(e) << i;
    }
    if (UNION && !last) {
      umask |= fa;
      if (mode != 2) continue;   // uniform: no ties to rank
      if (all_ties) {            // uniform: the ties need no order either
        umask |= fe;
        continue;
      }
      fa = 0ull;
    }
    // per round: the two counts packed as (A | E << 16); a wave's sums stay below 2^9 per half
    uint32_t ex[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const uint32_t c = static_cast<uint32_t>(__popcll((fa >> (4 * i)) & 0xFull)) |
                         (static_cast<uint32_t>(__popcll((fe >> (4 * i)) & 0xFull)) << 16);
      const uint32_t x = wave_inclusive_sum(c);
      if (lane == 63) {
        tot_a[i * NW + wave] = x & 0xFFFFu;
        tot_e[i * NW + wave] = x >> 16;
      }
      ex[i] = x - c;
    }
    __syncthreads();
    if (wave == 0) wave_exclusive_scan_lds(tot_a, R * NW, lane);
    if (wave == (NW > 1 ? 1 : 0)) wave_exclusive_scan_lds(tot_e, R * NW, lane);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < R; ++i) {
      uint32_t na = tot_a[i * NW + wave] + (ex[i] & 0xFFFFu);
      uint32_t ne = tot_e[i * NW + wave] + (ex[i] >> 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int bit = 4 * i + q;
        const int j = slot_of(bit);
        if ((fa >> bit) & 1ull) {
          const uint32_t o = na + min(ne, need);
          if (static_cast<int>(o) < p.b_cap) out[o] = j;
          ++na;
        } else if ((fe >> bit) & 1ull) {
          if (ne < need) {
            if (UNION && !last) {
              umask |= 1ull << bit;
            } else {
              const uint32_t o = na + ne;
              if (static_cast<int>(o) < p.b_cap) out[o] = j;
            }
          }
          ++ne;
        }
      }
    }
    if (UNION && !last) __syncthreads();  // tot_a / tot_e are rewritten by the next pass
  }
  for (int r = n_kept + tid; r < p.b_cap; r += NT) out[r] = -1;
  if (writer) p.n_kept[s] = n_kept;
}

// Caches past the register tiers (top-k and random past 32768 slots, the union past 65536;
// context lengths reach 128K tokens): the same rankings, threshold rule and ordered scan, with every step recomputing
// the keys from memory (a score load, or the Philox draw) instead of keeping them in registers.
// Steps: min/max (scores) and the 1024-bin histogram, the threshold bin's keys ranked in LDS (or,
// when crowded, OR/AND and 8-bit radix passes), then the ordered scan in chunks of 4 * NT slots
// in slot order with the kept and tied counts carried from chunk to chunk. The union (KIND 2)
// runs G + 1 such passes and keeps its union as a bit per slot in dynamic LDS (t_cap / 8 bytes).
constexpr int kStreamThreads = 1024;
static_assert(kSelectMaxSlotsUnion / 8 <= 32 * 1024, "union bits fit in 32 KB of LDS");

template <int KIND>
__global__ __launch_bounds__(kStreamThreads) void select_stream_kernel(const SelectParams p) {
  constexpr int NT = kStreamThreads;
  constexpr int NW = NT / 64;
  constexpr bool RANDOM = KIND == 1, UNION = KIND == 2;
  __shared__ __align__(16) uint32_t hist[kValueBins];
  __shared__ uint32_t red[2 * NW];
  __shared__ uint32_t wsum[2 * NW];
  __shared__ uint32_t found[3];
  __shared__ uint32_t n_members;
  __shared__ uint32_t kb[2];   // key interval of the threshold's bin
  extern __shared__ uint32_t ubits[];   // union: bit j set when slot j is in some head's top-k

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int head = blockIdx.x;
  const int h = head % p.H;
  const int s = (head / p.H) % p.S;
  const int l = head / (p.H * p.S);

  const int T = min(max(p.seq_len[s], 0), p.t_cap);
  const int P = min(max(p.prompt_len[s], 0), min(p.prompt_cap, T));
  const int B = p.budget;
  int32_t *out = p.kept + static_cast<size_t>(head) * p.b_cap;
  const bool writer = (l == 0 && h == 0 && tid == 0);

  if (T <= B) {  // nothing to compress: keep 0..T-1
    for (int r = tid; r < p.b_cap; r += NT) out[r] = r < T ? r : -1;
    if (writer) p.n_kept[s] = T;
    return;
  }
  const int Rw = min(p.recent, min(max(0, B - P), T - P));
  const int e_lo = P, e_hi = T - Rw;
  const int n_sel = max(0, B - P - Rw);
  const int n_kept = max(B, P);
  const int n_cand = e_hi - e_lo;
  const size_t slot0 = static_cast<size_t>(head) * p.t_cap;
  const uint32_t c1 = p.shared_draw ? 0u : (static_cast<uint32_t>(l) << 16) | static_cast<uint32_t>(h);
  const int passes = UNION ? (n_sel > 0 ? p.G : 0) + 1 : 1;
  const int k_head = UNION ? (p.k_per_head > 0 ? p.k_per_head : (n_sel + p.G - 1) / p.G) : 0;
  const int words = (T + 31) >> 5;
  if (UNION) {
    for (int w = tid; w < words; w += NT) ubits[w] = 0u;
    __syncthreads();
  }
  auto in_union = [&](int j) { return (ubits[j >> 5] >> (j & 31)) & 1u; };

#pragma unroll 1
  for (int pass = 0; pass < passes; ++pass) {
    const bool last = pass == passes - 1;
    // union, last pass: the union folded into the combined score's keys as in the register kernel
    bool long_union = false;
    if (UNION && last) {
      uint32_t cnt = 0u;
      for (int w = tid; w < words; w += NT) cnt += __popc(ubits[w]);
      cnt = wave_total(wave_inclusive_sum(cnt));
      if (lane == 0) red[wave] = cnt;
      __syncthreads();
      int n_union = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) n_union += static_cast<int>(red[w]);
      __syncthreads();
      long_union = n_union >= n_sel;
    }
    const float *row = nullptr;   // the scores this pass ranks by (not read by the random draw)
    if (!RANDOM) row = UNION && !last ? p.head_scores + (static_cast<size_t>(head) * p.G + pass) * p.t_cap
                                      : p.scores + slot0;
    auto key_of = [&](int j) -> uint32_t {  // j in [e_lo, e_hi)
      if (RANDOM) {
        const uint32_t c0 = p.pos ? static_cast<uint32_t>(p.pos[slot0 + j]) : static_cast<uint32_t>(j);
        return philox_word0(c0, c1, static_cast<uint32_t>(s), p.event, p.seed_lo, p.seed_hi);
      }
      const uint32_t k = order_key(row[j]);
      if (UNION && last) {
        const bool in_u = in_union(j);
        if (long_union && !in_u) return 0u;
        if (!long_union && in_u) return 0xFFFFFFFFu;
      }
      return k;
    };
    const int p_sel = UNION && !last ? k_head : n_sel;

    // mode: 0 = select none, 1 = select all candidates, 2 = threshold rule
    int mode;
    uint32_t thr = 0u, need = 0u;
    bool all_ties = false;  // every key equal to thr is taken
    if (p_sel <= 0 || n_cand <= 0) {
      mode = 0;
    } else if (p_sel >= n_cand) {
      mode = 1;
    } else {
      mode = 2;
      uint32_t remaining = static_cast<uint32_t>(p_sel);
      // member keys: those in the bin that holds the threshold (bins as in the register kernel),
      // or every candidate when the scores have no usable value range
      bool binned = RANDOM, ranked = false;
      uint32_t bsel = 0u, klo = 0u, khi = 0xFFFFFFFFu;   // key interval of the threshold's bin
      float fmin = 0.f, scale = 0.f;
      auto bin_of = [&](uint32_t k) { return RANDOM ? (k >> 22) : value_bin(k, fmin, scale); };
      if (!RANDOM) {
        uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
        for (int j = e_lo + tid; j < e_hi; j += NT) {
          const uint32_t k = key_of(j);
          if (k > kKeyNegInf && k < kKeyPosInf) {
            kmn = min(kmn, k);
            kmx = max(kmx, k);
          }
        }
        block_min_max<NT>(kmn, kmx, red);
        fmin = key_value(kmn);
        const float fmax = key_value(kmx);
        scale = static_cast<float>(kValueBins) / (fmax - fmin);
        binned = kmn < kmx && scale > 0.f && scale < 3.0e38f;
      }
      if (binned) {
        for (int i = tid; i < kValueBins; i += NT) hist[i] = 0u;
        if (tid == 0) n_members = 0u;
        __syncthreads();
        for (int j = e_lo + tid; j < e_hi; j += NT) atomicAdd(&hist[bin_of(key_of(j))], 1u);
        __syncthreads();
        if (wave == 0) find_bin<kValueBins>(hist, remaining, lane, found);
        __syncthreads();
        bsel = found[0];
        remaining -= found[1];
        bin_interval<RANDOM>(bsel, fmin, scale, wave, lane, kb);
        __syncthreads();  // `found` and `hist` are reused below; kb is written
        klo = kb[0];
        khi = kb[1];
        // a short member list is ranked directly (as in the register kernel)
        for (int j = e_lo + tid; j < e_hi; j += NT) {
          const uint32_t k = key_of(j);
          if (k >= klo && k <= khi) {
            const uint32_t at = atomicAdd(&n_members, 1u);
            if (at < member_cap<NT>()) hist[at] = k;
          }
        }
        __syncthreads();
        const uint32_t m = n_members;
        if (m <= member_cap<NT>()) {
          if (tid < 4) hist[m + tid] = 0u;
          __syncthreads();
          rank_members<NT>(hist, m, remaining, found);
          __syncthreads();
          thr = found[0];
          need = found[1];
          all_ties = found[2] == need;
          ranked = true;
        }
        __syncthreads();  // `found` and `hist` are reused below
      }
      auto member = [&](uint32_t k) { return !binned || (k >= klo && k <= khi); };
      if (!ranked) {
        uint32_t kor = 0u, kand = 0xFFFFFFFFu;
        for (int j = e_lo + tid; j < e_hi; j += NT) {
          const uint32_t k = key_of(j);
          if (member(k)) {
            kor |= k;
            kand &= k;
          }
        }
        block_or_and<NT>(kor, kand, red);
        const uint32_t diff = kor ^ kand;
        if (diff == 0u) {
          thr = kand;  // all member keys equal
        } else {
          const int top = 31 - __clz(diff);
          uint32_t mask = top == 31 ? 0u : ~((2u << top) - 1u);
          uint32_t prefix = kand & mask;
          for (int hi = top; hi >= 0;) {
            const int lo = hi >= 7 ? hi - 7 : 0;
            const uint32_t dmask = (1u << (hi - lo + 1)) - 1u;
            for (int i = tid; i < 256; i += NT) hist[i] = 0u;
            __syncthreads();
            for (int j = e_lo + tid; j < e_hi; j += NT) {
              const uint32_t k = key_of(j);
              if ((k & mask) == prefix && member(k)) atomicAdd(&hist[(k >> lo) & dmask], 1u);
            }
            __syncthreads();
            if (wave == 0) find_bin<256>(hist, remaining, lane, found);
            __syncthreads();
            prefix |= found[0] << lo;
            mask |= dmask << lo;
            remaining -= found[1];
            hi = lo - 1;
            __syncthreads();  // everyone has read `found` before the next pass may overwrite it
          }
          thr = prefix;
        }
        need = remaining;
      }
    }

    if (UNION && !last && (mode != 2 || all_ties)) {
      // a head's top-k needs no order: mark every candidate above (or at) the threshold
      for (int j = e_lo + tid; j < e_hi; j += NT) {
        const uint32_t k = mode == 2 ? key_of(j) : 0u;
        if (mode == 1 || (mode == 2 && k >= thr)) atomicOr(&ubits[j >> 5], 1u << (j & 31));
      }
      __syncthreads();
      continue;
    }

    // ordered scan: thread t takes slots c + 4t .. c + 4t + 3 of each chunk. The last pass writes
    // the kept list; a union head pass adds its top-k (ties to the lower slots) to the union.
    uint32_t carry_a = 0u, carry_e = 0u;  // unconditional / tied slots in earlier chunks
    for (int c = 0; c < T; c += 4 * NT) {
      const int j0 = c + 4 * tid;
      uint32_t fa = 0u, fe = 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = j0 + q;
        if (j >= T) break;
        const bool cnd = j >= e_lo && j < e_hi;
        bool a = last ? (!cnd || mode == 1) : (cnd && mode == 1), e = false;  // pins: last pass
        if (cnd && mode == 2) {
          const uint32_t k = key_of(j);
          a = k > thr;
          e = k == thr;
        }
        fa |= static_cast<uint32_t>(a) << q;
        fe |= static_cast<uint32_t>(e) << q;
      }
      const uint32_t cnt = static_cast<uint32_t>(__popc(fa)) | (static_cast<uint32_t>(__popc(fe)) << 16);
      const uint32_t x = wave_inclusive_sum(cnt);   // a wave's halves stay below 2^9
      if (lane == 63) {
        wsum[wave] = x & 0xFFFFu;
        wsum[NW + wave] = x >> 16;
      }
      __syncthreads();
      uint32_t na = carry_a + ((x - cnt) & 0xFFFFu), ne = carry_e + ((x - cnt) >> 16);
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        if (w < wave) {
          na += wsum[w];
          ne += wsum[NW + w];
        }
        carry_a += wsum[w];
        carry_e += wsum[NW + w];
      }
      __syncthreads();  // wsum is rewritten by the next chunk
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = j0 + q;
        if ((fa >> q) & 1u) {
          if (UNION && !last) {
            atomicOr(&ubits[j >> 5], 1u << (j & 31));
          } else {
            const uint32_t o = na + min(ne, need);
            if (o < static_cast<uint32_t>(p.b_cap)) out[o] = j;
          }
          ++na;
        } else if ((fe >> q) & 1u) {
          if (ne < need) {
            if (UNION && !last) {
              atomicOr(&ubits[j >> 5], 1u << (j & 31));
            } else {
              const uint32_t o = na + ne;
              if (o < static_cast<uint32_t>(p.b_cap)) out[o] = j;
            }
          }
          ++ne;
        }
      }
    }
    if (UNION && !last) __syncthreads();  // the union bits are complete before the next pass
  }
  for (int r = n_kept + tid; r < p.b_cap; r += NT) out[r] = -1;
  if (writer) p.n_kept[s] = n_kept;
}

// Recency+prompt ("Random Attention", section 4.1, the StreamingLLM-style diagnostic): the
// prompt and the n_kept - P latest slots, i.e. the evictable range's n_sel latest slots joined to
// the recent window. No scores are read; one thread per output entry.
__global__ __launch_bounds__(256) void recent_kernel(const SelectParams p, int chunks) {
  const int head = blockIdx.x / chunks;
  const int r = (blockIdx.x - head * chunks) * 256 + static_cast<int>(threadIdx.x);
  const int h = head % p.H;
  const int s = (head / p.H) % p.S;
  const int l = head / (p.H * p.S);
  const int T = min(max(p.seq_len[s], 0), p.t_cap);
  const int P = min(max(p.prompt_len[s], 0), min(p.prompt_cap, T));
  const bool compress = T > p.budget;
  const int n_kept = compress ? max(p.budget, P) : T;
  if (r == 0 && l == 0 && h == 0) p.n_kept[s] = n_kept;
  if (r >= p.b_cap) return;
  int v = -1;
  if (r < n_kept) v = (!compress || r < P) ? r : T - (n_kept - r);
  p.kept[static_cast<size_t>(head) * p.b_cap + r] = v;
}

// Audit of a kept list against the partition rules: one workgroup per head counts the entries
// that break them -- a kept index outside [0, T) or not above its predecessor, a prompt slot or
// recent-window slot missing from its place, an entry past n_kept that is not -1 -- and writes
// the count (0 = a valid keep-set), plus 1 if n_kept[s] differs from the partition's n_kept.
__global__ __launch_bounds__(256) void audit_kernel(const SelectParams p, int32_t *bad) {
  __shared__ int32_t red[4];
  const int head = blockIdx.x;
  const int s = (head / p.H) % p.S;
  const int T = min(max(p.seq_len[s], 0), p.t_cap);
  const int P = min(max(p.prompt_len[s], 0), min(p.prompt_cap, T));
  const int B = p.budget;
  const bool compress = T > B;
  const int Rw = compress ? min(p.recent, min(max(0, B - P), T - P)) : 0;
  const int n_kept = compress ? max(B, P) : T;
  const int nk = p.n_kept[s];
  const int32_t *kept = p.kept + static_cast<size_t>(head) * p.b_cap;
  int count = 0;
  for (int r = threadIdx.x; r < p.b_cap; r += 256) {
    const int v = kept[r];
    if (r >= n_kept) {
      count += v != -1;
    } else {
      const bool in_range = v >= 0 && v < T;
      const bool ascending = r == 0 || v > kept[r - 1];
      const bool prompt_ok = r >= P || v == r;
      const bool recent_ok = r < n_kept - Rw || v == T - (n_kept - r);
      count += !(in_range && ascending && prompt_ok && recent_ok);
    }
  }
  for (int off = 32; off >= 1; off >>= 1) count += __shfl_xor(count, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = count;
  __syncthreads();
  if (threadIdx.x == 0) bad[head] = red[0] + red[1] + red[2] + red[3] + (nk != n_kept);
}

// Only the (tier, ranking) pairs launch_select dispatches are instantiated.
template <int NT, int KPT, bool UNION>
hipError_t launch_cfg(const SelectParams &p, SelectKind kind, dim3 grid, hipStream_t st) {
  bool vec = (p.t_cap % 4 == 0) && ((reinterpret_cast<uintptr_t>(p.scores) & 15u) == 0);
  if constexpr (UNION) {
    vec = vec && ((reinterpret_cast<uintptr_t>(p.head_scores) & 15u) == 0);
    if (vec)
      hipLaunchKernelGGL((select_kernel<NT, KPT, 2, true>), grid, dim3(NT), 0, st, p);
    else
      hipLaunchKernelGGL((select_kernel<NT, KPT, 2, false>), grid, dim3(NT), 0, st, p);
  } else {
    if (kind == SelectKind::kRandom)
      hipLaunchKernelGGL((select_kernel<NT, KPT, 1, false>), grid, dim3(NT), 0, st, p);
    else if (vec)
      hipLaunchKernelGGL((select_kernel<NT, KPT, 0, true>), grid, dim3(NT), 0, st, p);
    else
      hipLaunchKernelGGL((select_kernel<NT, KPT, 0, false>), grid, dim3(NT), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_audit(const SelectParams &p, int32_t *bad, hipStream_t st) {
  const long long heads = static_cast<long long>(p.L) * p.S * p.H;
  if (heads <= 0) return hipSuccess;
  hipLaunchKernelGGL(audit_kernel, dim3(static_cast<unsigned>(heads)), dim3(256), 0, st, p, bad);
  return hipGetLastError();
}

hipError_t launch_select_recent(const SelectParams &p, hipStream_t st) {
  const long long heads = static_cast<long long>(p.L) * p.S * p.H;
  const int chunks = (p.b_cap + 255) / 256;
  if (heads <= 0) return hipSuccess;
  hipLaunchKernelGGL(recent_kernel, dim3(static_cast<unsigned>(heads * chunks)), dim3(256), 0, st, p, chunks);
  return hipGetLastError();
}

hipError_t launch_select(const SelectParams &p, SelectKind kind, hipStream_t st) {
  const long long heads = static_cast<long long>(p.L) * p.S * p.H;
  if (heads <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(heads));
  const int t = p.t_cap;
  if (kind == SelectKind::kUnion) {
    // The union's extra passes hold more registers: past 8192 slots it runs 512-thread tiers
    // (a 1024-thread workgroup is limited to 128 registers per lane); past 65536 slots, the
    // re-reading kernel with the union bits in dynamic LDS.
    if (t <= KV_UNION_STREAM_ABOVE) {
      if (t <= 256 * 4) return launch_cfg<256, 4, true>(p, kind, grid, st);
      if (t <= 256 * 16) return launch_cfg<256, 16, true>(p, kind, grid, st);
      if (t <= 256 * 32) return launch_cfg<256, 32, true>(p, kind, grid, st);
      if (t <= 512 * 32) return launch_cfg<512, 32, true>(p, kind, grid, st);
      if (t <= 512 * 64) return launch_cfg<512, 64, true>(p, kind, grid, st);
      if (t <= 1024 * 64) return launch_cfg<1024, 64, true>(p, kind, grid, st);
    }
    if (t > kSelectMaxSlotsUnion) return hipErrorInvalidValue;
    const size_t union_bytes = static_cast<size_t>((t + 31) / 32) * 4;
    hipLaunchKernelGGL(select_stream_kernel<2>, grid, dim3(kStreamThreads), union_bytes, st, p);
    return hipGetLastError();
  }
  if (t > KV_SELECT_STREAM_ABOVE) {
    if (kind == SelectKind::kRandom)
      hipLaunchKernelGGL(select_stream_kernel<1>, grid, dim3(kStreamThreads), 0, st, p);
    else
      hipLaunchKernelGGL(select_stream_kernel<0>, grid, dim3(kStreamThreads), 0, st, p);
    return hipGetLastError();
  }
  if (t <= 256 * 4) return launch_cfg<256, 4, false>(p, kind, grid, st);
  if (t <= 256 * 16) return launch_cfg<256, 16, false>(p, kind, grid, st);
  if (t <= 256 * 32) return launch_cfg<256, 32, false>(p, kind, grid, st);
  if (t <= 512 * 32) return launch_cfg<512, 32, false>(p, kind, grid, st);
#if KV_SELECT_WIDE
  if (t <= 512 * 64) return launch_cfg<512, 64, false>(p, kind, grid, st);
#else
  if (t <= 1024 * 32) return launch_cfg<1024, 32, false>(p, kind, grid, st);
#endif
#if KV_SELECT_STREAM_ABOVE > 32768
  if (t <= 1024 * 64) return launch_cfg<1024, 64, false>(p, kind, grid, st);
#endif
  return hipErrorInvalidValue;
}

}  // namespace kvevict

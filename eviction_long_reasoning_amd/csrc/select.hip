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
// One workgroup owns one (layer, seq, KV head). Its keys live in registers:
// thread t holds slot i*NT + t in round i, so every round is one coalesced
// 4-byte-per-lane load and the head's scores are read from HBM exactly once:
//  1. Keys: fp32 scores with NaN ranked as -inf (float comparisons give the
//     ranking, -0 equal to +0) or, for the random selector, word p mod 4 of
//     the Philox4x32-10 block at counter p div 4 (p the slot's position),
//     compared as uint32.
//  2. Listed path (selections of at most half the candidates): a cut below the
//     threshold -- from a sample of the scores (two rounds per thread, binned by
//     value) or, for uniform random words, from the selection's share -- is
//     checked by counting the keys at or above it (one ballot per round and
//     wave). When at least n_sel and at most the list's capacity pass, those
//     keys and their slots are copied to LDS in slot order, a 256-bin histogram
//     over the list finds the threshold's bin, and its members are ranked
//     directly: thr is the n_sel-th largest key, need the number of keys equal
//     to it that are taken. Placement then runs over the list alone: one
//     block-wide scan of per-thread (kept, tied) counts gives each kept entry
//     its output index. A cut that fails the count falls back to step 3.
//     Selections of more than half list the keys to evict the same way, with
//     the keys flipped (scores negated, random words complemented): the list
//     gives the threshold and how many of its ties are kept (the lowest slots),
//     and step 3's ballot placement writes the kept set.
//  3. Otherwise a 1024-bin LDS histogram over every key (scores binned by value
//     between the smallest and largest finite candidate, random keys by their
//     top 10 bits) finds the bin holding the n_sel-th largest key; its keys,
//     usually a few dozen, are listed in LDS and ranked directly. A crowded bin
//     instead goes through 8-bit radix passes over a 256-bin histogram, from
//     the highest bit where its keys differ (an OR/AND block reduction).
//     Placement without a sort: a selected evictable slot goes to P + (selected
//     slots before it), counted from one ballot per (round, wave) and the lanes
//     below it in its wave's ballot.
//  4. The prompt and the recent window go to their fixed places. Ties go to the
//     lower slot, and the kept list comes out in ascending order.
#include "kv_internal.hpp"

#include <type_traits>

namespace kvevict {
namespace {

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11): 10 rounds of two 32x32->64 products on counter
// words 0 and 2 with the published multipliers, the key advanced between
// rounds by the published Weyl constants. Returns the block's four words.
__device__ __forceinline__ uint4 philox_block(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
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
  return make_uint4(c0, c1, c2, c3);
}

// The draw of position p: word p mod 4 of the block with counter word 0 = p div 4, so one block
// serves four consecutive positions.
__device__ __forceinline__ uint32_t philox_draw(uint32_t p, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                uint32_t k1) {
  const uint4 b = philox_block(p >> 2, c1, c2, c3, k0, k1);
  const uint32_t w = p & 3u;
  return w == 0u ? b.x : w == 1u ? b.y : w == 2u ? b.z : b.w;
}

// The draws of a wave's GR rounds of 64 consecutive slots (round k, lane m: slot first + 64 k + m),
// pos[k] this lane's position in round k. When the positions run consecutively from a multiple of
// 4 over the whole group (always when they are the slots themselves and `first` is one), its 16 GR
// Philox blocks are drawn once each, GR / 4 per lane, and every lane takes its words from the lanes
// that drew them (round k, lane m: word m mod 4 of block 16 k + m / 4, drawn by lane
// 16 (k mod 4) + m / 4); otherwise every slot draws its own block. Call from wave-uniform control
// flow with every lane active.
template <int GR>
__device__ __forceinline__ void philox_group(uint32_t (&w)[GR], const uint32_t (&pos)[GR], int lane, uint32_t c1,
                                             uint32_t c2, uint32_t c3, uint32_t k0, uint32_t k1) {
  bool shared = false;
  if constexpr (GR % 4 == 0) {
    const uint32_t p0 = static_cast<uint32_t>(__shfl(static_cast<int>(pos[0]), 0, 64));
    bool run = (p0 & 3u) == 0u;
#pragma unroll
    for (int k = 0; k < GR; ++k) run = run && pos[k] == p0 + static_cast<uint32_t>(k * 64 + lane);
    shared = __builtin_amdgcn_ballot_w64(!run) == 0;
    if (shared) {
      uint4 blk[GR / 4];
#pragma unroll
      for (int b = 0; b < GR / 4; ++b)
        blk[b] = philox_block((p0 >> 2) + static_cast<uint32_t>(64 * b + lane), c1, c2, c3, k0, k1);
      const int sel = lane & 3;
#pragma unroll
      for (int k = 0; k < GR; ++k) {
        const int src = 16 * (k & 3) + (lane >> 2);
        const uint4 &bk = blk[k / 4];
        const uint32_t x = static_cast<uint32_t>(__shfl(static_cast<int>(bk.x), src, 64));
        const uint32_t y = static_cast<uint32_t>(__shfl(static_cast<int>(bk.y), src, 64));
        const uint32_t z = static_cast<uint32_t>(__shfl(static_cast<int>(bk.z), src, 64));
        const uint32_t v = static_cast<uint32_t>(__shfl(static_cast<int>(bk.w), src, 64));
        w[k] = sel == 0 ? x : sel == 1 ? y : sel == 2 ? z : v;
      }
    }
  }
  if (!shared) {
#pragma unroll
    for (int k = 0; k < GR; ++k) w[k] = philox_draw(pos[k], c1, c2, c3, k0, k1);
  }
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

// Lanes below this one whose bit is set in a wave-wide mask.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

constexpr uint32_t kKeyNegInf = 0x007FFFFFu;  // order_key(-inf)
constexpr uint32_t kKeyPosInf = 0xFF800000u;  // order_key(+inf)
constexpr int kValueBins = 1024;

// The fp32 value an order key stands for (inverse of order_key on non-NaN values).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Value binning of the threshold search: bins of equal width between the smallest and largest
// finite candidate, bin(v) = floor(v * scale + off) clamped to [0, kValueBins - 1] with
// off = -min * scale. One fused multiply-add, so the map never decreases as v grows: every bin's
// values form an interval. The clamp happens in floating point before the conversion (a NaN, -inf
// or negative value lands in bin 0, +inf in the last bin), so the conversion is always in range.
__device__ __forceinline__ uint32_t bin_of_value(float v, float scale, float off) {
  const float x = fminf(fmaxf(fmaf(v, scale, off), 0.f), static_cast<float>(kValueBins - 1));
  return static_cast<uint32_t>(x);
}
// The same map over order keys (all 2^32 of them: the patterns past +-inf go to the end bins). For a
// score x, bin_of_key(order_key(x)) == bin_of_value(x).
__device__ __forceinline__ uint32_t bin_of_key(uint32_t k, float scale, float off) {
  if (k <= kKeyNegInf) return 0u;
  if (k >= kKeyPosInf) return kValueBins - 1u;
  return bin_of_value(key_value(k), scale, off);
}

// bin_of_key never decreases as the key grows, so the keys of one bin form an interval. Run by one
// wave: the smallest key whose bin is at least `target`, or 2^32 when none is, by a 64-way search
// over the key space (at most seven rounds). It evaluates the same rounded expression as the
// histogram pass, so the interval test that replaces a second evaluation per key agrees with it key
// for key.
__device__ __forceinline__ uint64_t first_key_reaching(uint32_t target, float scale, float off, int lane) {
  uint64_t lo = 0, hi = uint64_t{1} << 32;   // keys below lo stay under target; hi reaches it (2^32: none)
  while (lo < hi) {
    const uint64_t step = (hi - lo + 63) >> 6;
    const uint64_t c = lo + static_cast<uint64_t>(lane) * step;
    const bool reach = c >= hi || bin_of_key(static_cast<uint32_t>(c), scale, off) >= target;
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
__device__ __forceinline__ void bin_interval(uint32_t b, float scale, float off, int wave, int lane,
                                             uint32_t *kb) {
  if (RANDOM) {
    if (wave == 0 && lane == 0) {
      kb[0] = b << 22;
      kb[1] = (b << 22) | 0x3FFFFFu;
    }
  } else if (wave < 2) {
    const uint64_t k = first_key_reaching(b + static_cast<uint32_t>(wave), scale, off, lane);
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

// Smallest and largest fp32 value over the workgroup; NaN inputs are ignored (fminf / fmaxf).
template <int NT>
__device__ __forceinline__ void block_fmin_fmax(float &mn, float &mx, float *lds /* 2*NT/64 */) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, off, 64));
    mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  }
  if (lane == 0) {
    lds[wave] = mn;
    lds[NW + wave] = mx;
  }
  __syncthreads();
  mn = INFINITY;
  mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    mn = fminf(mn, lds[i]);
    mx = fmaxf(mx, lds[NW + i]);
  }
  __syncthreads();  // lds may be reused right after
}

template <int NT>
__device__ __forceinline__ uint32_t block_sum(uint32_t x, uint32_t *lds /* NT/64 */) {
  constexpr int NW = NT / 64;
  x = wave_total(wave_inclusive_sum(x));
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = x;
  __syncthreads();
  uint32_t t = 0u;
#pragma unroll
  for (int i = 0; i < NW; ++i) t += lds[i];
  __syncthreads();
  return t;
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

// The listed path. A sample of the keys (one per thread) puts a cut below the threshold with high
// probability; the keys at or above it, typically 1.2-1.5 times the selection, are copied to LDS in
// slot order, and the threshold search and the ordered placement run over that list instead of over
// every key. The count of listed keys is checked before anything depends on the cut: a cut that
// leaves fewer keys than the selection, or more than the list holds, falls back to the search over
// all keys.
constexpr int kSampleBins = 256;
constexpr int kListBins = 256;
constexpr int kListMax = 6144;
constexpr int kStreamSamples = 4096;   // candidates sampled for a cut when the keys are not in registers
// A quarter of the tier's slots: a listing (of the selection, or of the keys to evict) never
// takes more than half the candidates, and a small list keeps the 256-thread tiers' LDS (and so
// their workgroups per CU) close to the histogram's.
template <int NT, int KPT>
constexpr int list_cap() { return NT * KPT / 4 < kListMax ? NT * KPT / 4 : kListMax; }

// Equal-width bins between a cut and the largest key, for any bin count (the clamp happens in
// floating point, so the conversion is always in range).
__device__ __forceinline__ uint32_t bin_clamped(float v, float scale, float off, int nbins) {
  const float x = fminf(fmaxf(fmaf(v, scale, off), 0.f), static_cast<float>(nbins - 1));
  return static_cast<uint32_t>(x);
}

// bin_clamped over order keys (the patterns below -inf go to bin 0, those from +inf up to the last).
__device__ __forceinline__ uint32_t bin_of_key_n(uint32_t k, float scale, float off, int nbins) {
  if (k <= kKeyNegInf) return 0u;
  if (k >= kKeyPosInf) return static_cast<uint32_t>(nbins - 1);
  return bin_clamped(key_value(k), scale, off, nbins);
}

// Run by every wave on its own (no barrier): with lane L owning bins PER*L ... PER*L + PER - 1 of
// an LDS histogram, the bin where the count from the top first reaches want_of(total) (0 when the
// total stays below it) and the count in the bins above it, both wave-uniform.
template <int NBINS, class Want>
__device__ __forceinline__ void wave_find_bin(const uint32_t *hist, Want want_of, int lane, uint32_t &bin,
                                              uint32_t &above, uint32_t &total) {
  constexpr int PER = NBINS / 64;
  uint32_t c[PER];
  uint32_t local = 0u;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    c[q] = hist[PER * lane + q];
    local += c[q];
  }
  const uint32_t incl = wave_inclusive_sum(local);
  total = wave_total(incl);
  const uint32_t want = want_of(total);
  uint32_t cum = total - incl;
  int mine = -1;
  uint32_t mine_above = 0u;
#pragma unroll
  for (int q = PER - 1; q >= 0; --q) {
    const uint32_t a = cum;
    cum += c[q];
    if (a < want && cum >= want) {
      mine = PER * lane + q;
      mine_above = a;
    }
  }
  const uint64_t m = __ballot(mine >= 0);
  if (m == 0ull) {
    bin = 0u;
    above = 0u;
    return;
  }
  const int src = __builtin_ctzll(m);
  bin = static_cast<uint32_t>(__builtin_amdgcn_readlane(mine, src));
  above = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(mine_above), src));
}

// 4-byte buffer load: the per-round offset rides in a scalar register, and reads past the
// resource's byte range return 0 without a memory access.
__device__ __forceinline__ uint32_t ld32(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

constexpr uint32_t kNoKey = 0x7FC00000u;   // quiet NaN: a score slot that takes no part

// The three rankings share one body. KIND 0 (top-k): keys are the fp32 scores. KIND 1 (random):
// keys are Philox words. KIND 2 (union, "TriAttention" blog, eviction step): G + 1 passes -- pass
// g < G ranks the evictable slots by query head g's own score and adds its top-k to a per-thread
// union bit mask; the last pass ranks by the combined score, inside the union when it holds at
// least n_sel slots, otherwise over the rest of the evictable range with the whole union kept.
// Every pass is a threshold search and an ordered placement; top-k and random run one pass.
//
// Layout: wave w owns the R*64 consecutive slots from w*R*64 on, and holds slot w*R*64 + i*64 + lane
// in round i (one key per lane and round). A wave's round is 64 consecutive slots read as one
// coalesced 256-byte load, and slot order is (wave, round, lane): a wave counts its kept slots in
// a scalar register as it goes, and only the NW wave totals are exchanged for the placement. R is
// a compile-time count the kernel picks per head (a quarter, half or all of the tier's KPT, the
// smallest whose NT*R slots reach the last evictable one), so every phase is straight-line code
// over registers: a uniform test per round, to skip rounds without evictable slots, cost more
// than the work it skipped.
//
// Slots that take no part (the prompt, the recent window, slots past the range) need no test
// either. Scores are held as fp32 with NaN replaced by -inf, so the float order is the ranking
// (-0 and +0 compare equal), and a NaN bit pattern marks a slot that takes no part -- it fails
// every comparison, fminf/fmaxf ignore it, and binning sends it to bin 0, which never moves the
// bin found for the threshold (bins are counted from the top and the threshold's keys are real).
// Random keys are uint32 words and a slot that takes no part holds 0: it is below or equal to
// every word, lands in bin 0 and matters only when the threshold lies in bin 0 -- then (rarely,
// and decided once per head) the member, tie and placement tests check the slot range as well.
//
// The prompt and recent window are placed arithmetically (kept[r] = r for r < P, the window after
// the selected slots), so the ordered placement only ranks evictable slots: a selected slot's
// output index is P + (selected slots before it).
struct SelectSmem {
  uint32_t *hist;     // kValueBins words; also the member list
  float *fred;        // 2 * NW
  uint32_t *red;      // 2 * NW
  uint32_t *cnt_a;    // NW: per wave, evictable slots kept outright
  uint32_t *cnt_e;    // NW: per wave, slots equal to the threshold
  uint32_t *found;    // 3
  uint32_t *n_members;
  // the listed path
  uint32_t *shist;    // kSampleBins: the sample's value histogram
  uint32_t *mlist;    // kValueBins: the threshold bin's members, zero beyond the last
  uint32_t *cnt_l;    // NW: per wave, listed keys, then packed placement counts
  uint32_t *lkey;     // list_cap: key bits of the listed slots, in slot order (scores as fp32 bits,
                      // random keys as the word)
  uint32_t *lslot;    // list_cap: their slots (same index: one address, two immediate offsets)
  int list_cap;
};

struct SelectHead {
  int head, l, h, s;
  int P, e_lo, e_hi, n_sel, n_cand;
  int32_t *out;
};

// The listed path's cut for Philox words: the p_sel-th largest of n_valid uniform words sits near
// 2^32 (1 - p_sel / n_valid); the cut leaves about four standard deviations more. At least 1, so
// a slot that takes no part (word 0) is never listed.
__device__ __forceinline__ uint32_t random_cut(int p_sel, int n_valid) {
  const float want = static_cast<float>(p_sel) + 4.f * sqrtf(static_cast<float>(p_sel)) + 16.f;
  if (!(want < static_cast<float>(n_valid))) return 1u;
  const double c = 4294967296.0 * (1.0 - static_cast<double>(want) / static_cast<double>(n_valid));
  return c > 1.0 ? static_cast<uint32_t>(c) : 1u;
}

// Whether p_sel of n_valid keys can be listed: at most half the candidates (more than half are
// listed from the other end, as the keys to evict), and room in a list of list_cap for the cut's
// margin.
__device__ __forceinline__ bool listable(int p_sel, int n_valid, int list_cap) {
  return p_sel > 0 && p_sel < n_valid && 2 * p_sel <= n_valid && p_sel + p_sel / 8 + 64 <= list_cap;
}

// The threshold over a list of `total` keys in sm.lkey (scores as fp32 bits between lo and hi,
// random words at or above cut_k): a kListBins histogram (sm.hist, which must be zero), the bin
// of the p_sel-th largest found by every wave, its members (sm.mlist, zero beyond any earlier
// member list; *sm.n_members zero) ranked directly. False, with nothing decided, when the score
// range is unusable or the bin is too crowded to rank; the caller then takes the full path.
template <int NT, bool RANDOM>
__device__ __forceinline__ bool list_threshold(const SelectSmem &sm, uint32_t total, uint32_t p_sel, float lo, float hi,
                               uint32_t cut_k, uint32_t &thr, uint32_t &need, bool &all_ties) {
  const int tid = threadIdx.x, lane = tid & 63;
  const float scale2 = static_cast<float>(kListBins) / (hi - lo), off2 = -lo * scale2;
  if (!RANDOM && !(hi > lo && scale2 > 0.f && scale2 < 3.0e38f && fabsf(off2) < 3.0e38f)) return false;
  const uint32_t span = 0xFFFFFFFFu - cut_k;
  const int bits = span ? 32 - __clz(span) : 0;
  const int shift = bits > 8 ? bits - 8 : 0;
  auto lbin = [&](uint32_t k) {
    return RANDOM ? (k - cut_k) >> shift : bin_clamped(__uint_as_float(k), scale2, off2, kListBins);
  };
  for (uint32_t e = tid; e < total; e += NT) atomicAdd(&sm.hist[lbin(sm.lkey[e])], 1u);
  __syncthreads();
  uint32_t b, above, tot;
  wave_find_bin<kListBins>(sm.hist, [&](uint32_t) { return p_sel; }, lane, b, above, tot);
  const uint32_t rem = p_sel - above;
  for (uint32_t e = tid; e < total; e += NT) {
    const uint32_t k = sm.lkey[e];
    if (lbin(k) == b) {
      const uint32_t at = atomicAdd(sm.n_members, 1u);
      if (at < member_cap<NT>()) sm.mlist[at] = RANDOM ? k : order_key(__uint_as_float(k));
    }
  }
  __syncthreads();
  const uint32_t m = *sm.n_members;
  if (m > member_cap<NT>()) return false;
  rank_members<NT>(sm.mlist, m, rem, sm.found);   // entries past m are still zero
  __syncthreads();
  thr = sm.found[0];
  need = sm.found[1];
  all_ties = sm.found[2] == need;
  return true;
}

// Placement from a list in slot order: thread t takes a contiguous run of list entries, so one
// block-wide scan of its (kept outright, tied) counts orders every output. Scores compare as fp32
// against the threshold's value (-0 equals +0, as for order keys).
template <int NT, bool RANDOM>
__device__ __forceinline__ void list_place(const SelectSmem &sm, uint32_t n, uint32_t thr, uint32_t need, bool all_ties, int P,
                           int32_t *out, int b_cap) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t per = (n + NT - 1) / NT;
  const uint32_t e0 = min(n, static_cast<uint32_t>(tid) * per), e1 = min(n, e0 + per);
  const float thr_v = key_value(thr);
  auto is_a = [&](uint32_t k) {
    if (RANDOM) return all_ties ? k >= thr : k > thr;
    return all_ties ? __uint_as_float(k) >= thr_v : __uint_as_float(k) > thr_v;
  };
  auto is_t = [&](uint32_t k) { return RANDOM ? k == thr : __uint_as_float(k) == thr_v; };
  uint32_t ca = 0u, ct = 0u;
  for (uint32_t e = e0; e < e1; ++e) {
    const uint32_t k = sm.lkey[e];
    ca += is_a(k) ? 1u : 0u;
    ct += (!all_ties && is_t(k)) ? 1u : 0u;
  }
  const uint32_t packed = ca | (ct << 16);   // both at most kListMax
  const uint32_t incl = wave_inclusive_sum(packed);
  if (lane == 63) sm.cnt_l[wave] = incl;
  __syncthreads();
  uint32_t below = incl - packed;
  for (int w = 0; w < wave; ++w) below += sm.cnt_l[w];
  uint32_t ra = below & 0xFFFFu, re = below >> 16;
  for (uint32_t e = e0; e < e1; ++e) {
    const uint32_t k = sm.lkey[e];
    uint32_t o = 0xFFFFFFFFu;
    if (is_a(k)) {
      o = static_cast<uint32_t>(P) + ra + min(re, need);
      ++ra;
    } else if (!all_ties && is_t(k)) {
      if (re < need) o = static_cast<uint32_t>(P) + ra + re;
      ++re;
    }
    if (o < static_cast<uint32_t>(b_cap)) out[o] = static_cast<int32_t>(sm.lslot[e]);
  }
}

// The smallest key whose bin is at least `target` (2^32 when none is), run by one wave. The bin
// boundary sits near the value (target - off) / scale; one probe of the 64 keys around that
// value's key settles it when the boundary lies among them (lane 0 below, some lane at or above:
// the bin never decreases with the key, so the first lane that reaches is the boundary).
// Otherwise, or for a boundary near an infinite or cancelling estimate, the 64-way search over the
// whole key space.
__device__ __forceinline__ uint64_t first_key_reaching_near(uint32_t target, float scale, float off, int lane) {
  if (target == 0u) return 0u;
  if (target >= static_cast<uint32_t>(kValueBins)) return uint64_t{1} << 32;
  const float v = (static_cast<float>(target) - off) / scale;
  if (v > -INFINITY && v < INFINITY) {
    const uint32_t k0 = order_key(v);
    if (k0 >= 32u && k0 <= 0xFFFFFFFFu - 32u) {
      const uint32_t c = k0 - 32u + static_cast<uint32_t>(lane);
      const uint64_t m = __ballot(bin_of_key(c, scale, off) >= target);
      if (m != 0ull && !(m & 1ull)) return static_cast<uint64_t>(k0 - 32u) + static_cast<uint64_t>(__builtin_ctzll(m));
    }
  }
  return first_key_reaching(target, scale, off, lane);
}

template <int NT, int R, int KIND>
__device__ __forceinline__ void select_rounds(const SelectParams &p, const SelectSmem &sm, const SelectHead &hd) {
  constexpr int NW = NT / 64;
  constexpr bool RANDOM = KIND == 1, UNION = KIND == 2;
  static_assert(R <= 32, "one union bit per round");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int e_lo = hd.e_lo, e_hi = hd.e_hi, n_sel = hd.n_sel, n_cand = hd.n_cand, P = hd.P;
  uint32_t *hist = sm.hist;
  uint32_t *found = sm.found;
  const size_t slot0 = static_cast<size_t>(hd.head) * p.t_cap;
  // Slot of round 0 for this lane, as a phase sees it: the thread index passes through an empty
  // asm at the start of each phase, so slots and lane tests are derived where they are used. Left
  // free, the compiler derives every round's slot and mask once and holds them across the kernel,
  // more registers than the keys themselves.
  auto slot_base = [&]() {
    int t = tid;
    asm volatile("" : "+v"(t));
    return (t & ~63) * R + (t & 63);
  };
  // slot j0 + i*64 lies in [e_lo, e_hi): one unsigned comparison, no branch
  auto evictable = [&](int j0, int i) {
    return static_cast<uint32_t>(j0 + i * 64 - e_lo) < static_cast<uint32_t>(n_cand);
  };

  uint32_t key[R];
  auto fkey = [&](int i) { return __uint_as_float(key[i]); };
  // order key of round i's key (scores: order_key of the value; random: the word itself)
  auto okey = [&](int i) { return RANDOM ? key[i] : order_key(fkey(i)); };

  if (RANDOM) {
    // A draw costs about a hundred instructions: groups of rounds with no evictable slot in this
    // wave are skipped (a wave-uniform test per group), the rest run straight-line so that the
    // group's draws interleave.
    constexpr int GR = R < 8 ? R : 8;
    const uint32_t c1 =
        p.shared_draw ? 0u : (static_cast<uint32_t>(hd.l + p.layer_base) << 16) | static_cast<uint32_t>(hd.h);
    const __amdgpu_buffer_rsrc_t rp = rsrc_of(p.pos ? p.pos + slot0 : p.seq_len, p.pos ? e_hi * 4 : 0);
    const int j0 = slot_base();
#pragma unroll
    for (int g = 0; g < R; g += GR) {
      const int first = (wave * R + g) * 64, end = first + GR * 64;   // the group's slots in this wave
#pragma unroll
      for (int i = g; i < g + GR; ++i) key[i] = 0u;
      if (end > e_lo && first < e_hi) {
        uint32_t c0s[GR];   // the positions of this lane's slots in the group
#pragma unroll
        for (int k = 0; k < GR; ++k) {
          const int j = j0 + (g + k) * 64;
          c0s[k] = p.pos ? ld32(rp, j * 4, 0) : static_cast<uint32_t>(j);
        }
        uint32_t w[GR];
        philox_group<GR>(w, c0s, lane, c1, static_cast<uint32_t>(hd.s), p.event, p.seed_lo, p.seed_hi);
#pragma unroll
        for (int k = 0; k < GR; ++k) key[g + k] = evictable(j0, g + k) ? w[k] : 0u;
      }
    }
  }

  const int passes = UNION ? p.G + 1 : 1;
  const int k_head = UNION ? (p.k_per_head > 0 ? p.k_per_head : (n_sel + p.G - 1) / p.G) : 0;
  uint32_t umask = 0u;   // union: bit i set when round i's slot is in some query head's top-k

#pragma unroll 1
  for (int pass = 0; pass < passes; ++pass) {
    const bool last = pass == passes - 1;
    if (!RANDOM) {
      const float *row = UNION && !last ? p.head_scores + (static_cast<size_t>(hd.head) * p.G + pass) * p.t_cap
                                        : p.scores + slot0;
      // the offset rides in the per-lane operand and the instruction's offset, which the buffer's
      // range check covers: slots at or past e_hi read 0 without a memory access
      const __amdgpu_buffer_rsrc_t rs = rsrc_of(row, e_hi * 4);
      const int j0 = slot_base();
#pragma unroll
      for (int i = 0; i < R; ++i) key[i] = ld32(rs, j0 * 4 + i * 256, 0);
      const int j1 = slot_base();
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const float x = fmaxf(__uint_as_float(key[i]), -INFINITY);   // NaN ranks as -inf
        key[i] = evictable(j1, i) ? __float_as_uint(x) : kNoKey;
      }
    }
    int p_sel = n_sel, n_valid = n_cand;
    bool short_union = false;
    if (UNION && !last) {
      p_sel = k_head;
    } else if (UNION) {
      const int n_union = static_cast<int>(block_sum<NT>(static_cast<uint32_t>(__builtin_popcount(umask)), sm.red));
      // A long union (>= n_sel slots) is ranked alone; a short one is kept whole and the rest of the
      // evictable range ranks for the places that remain.
      short_union = n_union < n_sel;
      const uint32_t drop = short_union ? umask : ~umask;
#pragma unroll
      for (int i = 0; i < R; ++i)
        if ((drop >> i) & 1u) key[i] = kNoKey;
      if (short_union) {
        p_sel = n_sel - n_union;
        n_valid = n_cand - n_union;
      } else {
        n_valid = n_union;
      }
    }

    // ---- threshold: thr = the p_sel-th largest valid key; `need` of the keys equal to it are taken
    // mode: 0 = take none, 1 = take every valid key, 2 = threshold rule
    const int mode = p_sel <= 0 ? 0 : (p_sel >= n_valid ? 1 : 2);
    uint32_t thr = 0u, need = 0u;   // thr as an order key (scores) or a word (random)
    bool all_ties = true;           // every key equal to thr is taken
    bool careful = false;           // random keys: the slot range decides membership, ties, placement
    bool listed = false;            // the threshold came from the list, which is still in LDS
    uint32_t n_list = 0u;
    if (mode == 2) {
      uint32_t remaining = static_cast<uint32_t>(p_sel);
      bool binned = RANDOM, ranked = false;
      float scale = 0.f, off = 0.f;
      float mn = INFINITY, mx = -INFINITY;
      // the listed path's LDS starts cleared (its readers in an earlier pass are behind a barrier;
      // the barriers of the min/max reduction, or of the count below, order this before any use)
      for (int i = tid; i < kValueBins; i += NT) {
        hist[i] = 0u;
        sm.mlist[i] = 0u;
      }
      for (int i = tid; i < kSampleBins; i += NT) sm.shist[i] = 0u;
      if (tid == 0) *sm.n_members = 0u;
      if (!RANDOM) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
          mn = fminf(mn, fkey(i));
          mx = fmaxf(mx, fkey(i));
        }
        block_fmin_fmax<NT>(mn, mx, sm.fred);
        if (!(mn > -INFINITY && mx < INFINITY)) {   // an infinite key: the range of the finite ones
          mn = INFINITY;
          mx = -INFINITY;
#pragma unroll
          for (int i = 0; i < R; ++i) {
            const float x = fkey(i);
            if (x > -INFINITY && x < INFINITY) {
              mn = fminf(mn, x);
              mx = fmaxf(mx, x);
            }
          }
          block_fmin_fmax<NT>(mn, mx, sm.fred);
        }
        scale = static_cast<float>(kValueBins) / (mx - mn);
        off = -mn * scale;
        binned = mn < mx && scale > 0.f && scale < 3.0e38f && fabsf(off) < 3.0e38f;
      }

      // ---- listed path: cut, count, list, then the threshold over the list
      // the `want` largest keys (the selection, or the count to evict when the keys are flipped)
      auto try_list = [&](int want) __attribute__((always_inline)) -> bool {
        float cut_f = -INFINITY;   // scores: list x >= cut_f (NaN marks never pass)
        uint32_t cut_k = 1u;       // random: list words >= cut_k (slots that take no part hold 0)
        if (RANDOM) {
          cut_k = random_cut(want, n_valid);
        } else {
          // two keys per thread (rounds R/4 and 3R/4: two blocks of 64 consecutive slots per wave,
          // spread evenly over the head) into kSampleBins value bins; the cut is one bin below where
          // the count from the top reaches the sample's expected share of `want` plus three standard
          // deviations. The rounds are fixed: a per-lane choice of round would index the key array.
          const float sscale = static_cast<float>(kSampleBins) / (mx - mn), soff = -mn * sscale;
          constexpr int kS0 = R >= 4 ? R / 4 : 0, kS1 = R >= 4 ? 3 * R / 4 : R - 1;
          const float sx0 = fkey(kS0), sx1 = fkey(kS1);
          if (sx0 == sx0) atomicAdd(&sm.shist[bin_clamped(sx0, sscale, soff, kSampleBins)], 1u);
          if (kS1 != kS0 && sx1 == sx1) atomicAdd(&sm.shist[bin_clamped(sx1, sscale, soff, kSampleBins)], 1u);
          __syncthreads();
          uint32_t bc, above_s, n_s;
          wave_find_bin<kSampleBins>(sm.shist, [&](uint32_t tot) {
            const float lam = static_cast<float>(want) * static_cast<float>(tot) / static_cast<float>(n_valid);
            return static_cast<uint32_t>(lam + 3.f * sqrtf(lam) + 4.f);
          }, lane, bc, above_s, n_s);
          if (bc > 1u) cut_f = (static_cast<float>(bc - 1u) - soff) / sscale;
        }
        auto pass_cut = [&](int i) { return RANDOM ? key[i] >= cut_k : fkey(i) >= cut_f; };
        uint32_t cnt = 0u;
#pragma unroll
        for (int i = 0; i < R; ++i) cnt += static_cast<uint32_t>(__popcll(__ballot(pass_cut(i))));
        if (lane == 0) sm.cnt_l[wave] = cnt;
        __syncthreads();
        uint32_t total = 0u, base = 0u;
        for (int w = 0; w < NW; ++w) {
          const uint32_t c = sm.cnt_l[w];
          if (w < wave) base += c;
          total += c;
        }
        if (total < static_cast<uint32_t>(want) || total > static_cast<uint32_t>(sm.list_cap)) return false;
        // bins over the listed range: scores by value between the cut (or the smallest finite key)
        // and the largest; random words by their offset above the cut
        const float lo = cut_f > -INFINITY ? cut_f : mn;
        if (!RANDOM && !(mx > lo)) return false;
        {
          const int j0 = slot_base();
#pragma unroll
          for (int i = 0; i < R; ++i) {
            const bool m = pass_cut(i);
            const uint64_t b = __ballot(m);
            if (m) {
              const uint32_t at = base + lanes_below(b);
              sm.lkey[at] = key[i];
              sm.lslot[at] = static_cast<uint32_t>(j0 + i * 64);
            }
            base += static_cast<uint32_t>(__popcll(b));
          }
        }
        __syncthreads();
        if (!list_threshold<NT, RANDOM>(sm, total, static_cast<uint32_t>(want), lo, mx, cut_k, thr, need, all_ties))
          return false;
        n_list = total;
        return true;
      };
      // More than half selected: the same listing from the other end. The keys are flipped (scores
      // negated, random words complemented) so the q = n_valid - p_sel lowest come first; the list
      // gives the q-th lowest key, the number of keys equal to it (all of them are listed) and how
      // many of those the q lowest take. The kept set is then every key above it and, of the keys
      // equal to it, the lowest-slot (ties - taken), placed by the ordered scan below.
      bool flipped = false;
      const int q_evict = n_valid - p_sel;
      auto flip_keys = [&]() {
        const int jf = slot_base();
#pragma unroll
        for (int i = 0; i < R; ++i) key[i] = RANDOM ? (evictable(jf, i) ? ~key[i] : 0u) : key[i] ^ 0x80000000u;
      };
      const bool list_top = binned && listable(p_sel, n_valid, sm.list_cap);
      const bool list_low = !UNION && !list_top && binned && listable(q_evict, n_valid, sm.list_cap);
      const float mn0 = mn, mx0 = mx;
      if (list_low) {
        flip_keys();
        mn = -mx0;
        mx = -mn0;
      }
      if (list_top || list_low) {   // one call site: the listing is inlined once
        const bool ok = try_list(list_low ? q_evict : p_sel);
        listed = list_top && ok;
        flipped = list_low && ok;
      }
      if (list_low) {
        mn = mn0;
        mx = mx0;
        flip_keys();
      }
      if (flipped) {
        const uint32_t ties_at = sm.found[2];   // keys equal to the q-th lowest (rank_members' count)
        thr = RANDOM ? ~thr : order_key(-key_value(thr));
        need = ties_at - need;                  // the ties kept: those the q lowest leave
        all_ties = need == ties_at;
        careful = RANDOM && thr == 0u;          // word 0 is also the mark of a slot that takes no part
      }
      if (!listed && !flipped) {
      __syncthreads();   // the previous pass's readers of hist are done
      // valid: the key takes part (scores: not the NaN mark; random: the slot range)
      auto valid = [&](int i, int j0) {
        if (RANDOM) return evictable(j0, i);
        return fkey(i) == fkey(i);
      };
      // exact radix passes over the keys member(i, j0) still has to order
      auto radix = [&](auto member) {
        uint32_t kor = 0u, kand = 0xFFFFFFFFu;
        const int j0 = slot_base();
#pragma unroll
        for (int i = 0; i < R; ++i)
          if (member(i, j0)) {
            kor |= okey(i);
            kand &= okey(i);
          }
        block_or_and<NT>(kor, kand, sm.red);
        const uint32_t diff = kor ^ kand;
        if (diff == 0u) {
          thr = kand;   // all member keys equal
        } else {
          const int top = 31 - __clz(diff);
          uint32_t mask = top == 31 ? 0u : ~((2u << top) - 1u);
          uint32_t prefix = kand & mask;
          for (int hi = top; hi >= 0;) {
            const int lo = hi >= 7 ? hi - 7 : 0;
            const uint32_t dmask = (1u << (hi - lo + 1)) - 1u;
            for (int i = tid; i < 256; i += NT) hist[i] = 0u;
            __syncthreads();
            const int j1 = slot_base();
#pragma unroll
            for (int i = 0; i < R; ++i)
              if (member(i, j1) && (okey(i) & mask) == prefix) atomicAdd(&hist[(okey(i) >> lo) & dmask], 1u);
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
        all_ties = false;
      };
      if (binned) {
        for (int i = tid; i < kValueBins; i += NT) hist[i] = 0u;
        if (tid == 0) *sm.n_members = 0u;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < R; ++i)   // NaN marks and random 0 marks land in bin 0
          atomicAdd(&hist[RANDOM ? key[i] >> 22 : bin_of_value(fkey(i), scale, off)], 1u);
        __syncthreads();
        if (wave == 0) find_bin<kValueBins>(hist, remaining, lane, found);
        __syncthreads();
        const uint32_t b = found[0];
        remaining -= found[1];
        careful = RANDOM && b == 0u;
        // Members of the threshold's bin: a key-interval test. Random keys' bins are their top 10
        // bits; for scores every wave finds the bin's bounds itself (no barrier).
        uint32_t klo, khi;
        if (RANDOM) {
          klo = b << 22;
          khi = (b << 22) | 0x3FFFFFu;
        } else {
          klo = static_cast<uint32_t>(first_key_reaching_near(b, scale, off, lane));
          khi = static_cast<uint32_t>(first_key_reaching_near(b + 1u, scale, off, lane) - 1u);
        }
        const float flo = key_value(max(klo, kKeyNegInf)), fhi = key_value(min(khi, kKeyPosInf));
        auto member = [&](int i, int j0) {
          if (RANDOM) return key[i] >= klo && key[i] <= khi && (!careful || valid(i, j0));
          return fkey(i) >= flo && fkey(i) <= fhi;
        };
        // The bin usually holds a few dozen keys: list them in LDS (hist is free once every wave
        // has read `found`) and rank them directly.
        __syncthreads();
        const int jm = slot_base();
#pragma unroll
        for (int i = 0; i < R; ++i) {
          if (member(i, jm)) {
            const uint32_t at = atomicAdd(sm.n_members, 1u);
            if (at < member_cap<NT>()) hist[at] = okey(i);
          }
        }
        __syncthreads();
        const uint32_t m = *sm.n_members;
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
        if (!ranked) radix(member);   // a crowded bin: exact radix passes over its keys
      } else {
        // no usable value range (all finite candidates equal, or none finite): radix passes over
        // every valid key
        radix(valid);
      }
      }
    }

    // ---- placement from the list (top-k and random)
    if (!UNION && listed) {
      list_place<NT, RANDOM>(sm, n_list, thr, need, all_ties, P, hd.out, p.b_cap);
      continue;
    }

    // ---- placement. A: kept outright (above the threshold, or equal to it when every tie is
    // taken, or a short union's own slot); E: equal to the threshold, kept while fewer than `need`
    // earlier (lower-slot) ties are. A is one comparison against a bound: scores x >= a_f (mode 2:
    // thr, or the next key up when ties are ranked; mode 1: -inf; mode 0: NaN), random keys
    // key + a_add > a_thr in 64 bits.
    const bool ties = mode == 2 && !all_ties;
    const float thr_f = key_value(thr);
    const float a_f = mode == 2 ? key_value(all_ties ? thr : thr + 1u) : (mode == 1 ? -INFINITY : __uint_as_float(kNoKey));
    const uint64_t a_thr = mode == 2 ? thr : (mode == 1 ? 0ull : 0xFFFFFFFFull);
    const uint64_t a_add = mode == 2 ? (all_ties ? 1ull : 0ull) : (mode == 1 ? 1ull : 0ull);
    const uint32_t extra = UNION && last && short_union ? umask : 0u;
    auto place = [&](auto careful_t) {
      constexpr bool CAREFUL = decltype(careful_t)::value;
      auto in_range = [&](int i, int j0) { return !CAREFUL || evictable(j0, i); };
      auto is_a = [&](int i, int j0) {
        bool a;
        if (RANDOM) a = static_cast<uint64_t>(key[i]) + a_add > a_thr && in_range(i, j0);
        else a = fkey(i) >= a_f;
        if (UNION) a = a || ((extra >> i) & 1u);
        return a;
      };
      auto is_e = [&](int i, int j0) { return RANDOM ? (key[i] == thr && in_range(i, j0)) : fkey(i) == thr_f; };
      if (UNION && !last && !ties) {   // a query head's top-k needs no order
        const int j0 = slot_base();
#pragma unroll
        for (int i = 0; i < R; ++i)
          if (is_a(i, j0)) umask |= 1u << i;
        return;
      }
      // this wave's totals, then the totals of the lower waves
      uint32_t ta = 0u, te = 0u;
      const int jc = slot_base();
#pragma unroll
      for (int i = 0; i < R; ++i) {
        ta += static_cast<uint32_t>(__popcll(__ballot(is_a(i, jc))));
        if (ties) te += static_cast<uint32_t>(__popcll(__ballot(is_e(i, jc))));
      }
      __syncthreads();   // the previous pass's readers of cnt_a / cnt_e are done
      if (lane == 0) {
        sm.cnt_a[wave] = ta;
        sm.cnt_e[wave] = te;
      }
      __syncthreads();
      const uint32_t va = lane < NW ? sm.cnt_a[lane] : 0u, ve = lane < NW ? sm.cnt_e[lane] : 0u;
      uint32_t na = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wave_inclusive_sum(va) - va), wave));
      uint32_t ne = ties ? static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wave_inclusive_sum(ve) - ve), wave)) : 0u;
      const int jp = slot_base();
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const bool a = is_a(i, jp);
        const uint64_t ba = __ballot(a);
        const uint32_t ra = na + lanes_below(ba);   // kept-outright slots before this one
        na += static_cast<uint32_t>(__popcll(ba));
        uint32_t re = 0u;
        bool e = false;
        if (ties) {
          e = is_e(i, jp);
          const uint64_t be = __ballot(e);
          re = ne + lanes_below(be);                // tied slots before this one
          ne += static_cast<uint32_t>(__popcll(be));
        }
        const bool take_e = e && re < need;
        if (UNION && !last) {
          if (a || take_e) umask |= 1u << i;
        } else if (a || take_e) {
          const uint32_t o = static_cast<uint32_t>(P) + ra + (a ? min(re, need) : re);
          if (o < static_cast<uint32_t>(p.b_cap)) hd.out[o] = jp + i * 64;
        }
      }
    };
    if (RANDOM && careful) place(std::true_type{});
    else place(std::false_type{});
  }
}

// Split draw, for random selection over batches with few heads and long caches: split_chunks
// workgroups per head each draw kSplitChunk consecutive candidates' Philox words, so the draw (the
// bulk of the work) runs on many CUs instead of one. Every chunk workgroup takes the same cut (the
// selection's share, as in the register kernel), lists its candidates at or above it in slot order
// into the workspace and writes their count. The head's ranking workgroup (select_kernel) then
// gathers the lists in chunk order, which is slot order, and ranks and places over them; when they
// do not fit, or the threshold's bin is too crowded, it takes its full path over every key instead.
// Top-k selection was measured without a gain from the same split (its chunk and ranking kernels
// took 5.3 + 8.4 us against 12-13 us for one workgroup per head on 8 heads of 32768 slots: the
// ranking workgroup's chain of dependent loads and barriers costs what the split saves), so it keeps
// one workgroup per head.
constexpr int kSplitThreads = 256;
constexpr int kSplitMaxChunks = kSelectMaxSlots / kSplitChunk;   // 16

__global__ __launch_bounds__(kSplitThreads) void select_split_kernel(const SelectParams p) {
  constexpr int NT = kSplitThreads, NW = NT / 64, R = kSplitChunk / NT;
  __shared__ uint32_t cnt[NW];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int chunk = blockIdx.x % p.split_chunks;
  const int head = blockIdx.x / p.split_chunks;
  const int h = head % p.H, s = (head / p.H) % p.S, l = head / (p.H * p.S);
  const int T = __builtin_amdgcn_readfirstlane(min(max(p.seq_len[s], 0), p.t_cap));
  const int P = __builtin_amdgcn_readfirstlane(min(max(p.prompt_len[s], 0), min(p.prompt_cap, T)));
  const int B = p.budget;
  uint32_t *count = p.split_count + static_cast<size_t>(head) * p.split_chunks + chunk;
  const int Rw = min(p.recent, min(max(0, B - P), T - P));
  const int e_lo = P, e_hi = T - Rw;
  const int n_sel = max(0, B - P - Rw), n_cand = e_hi - e_lo;
  const int c_lo = e_lo + chunk * kSplitChunk;
  // heads the ranking workgroup does not list, and chunks past the evictable range, list nothing
  if (T <= B || !listable(n_sel, n_cand, p.split_list_cap) || c_lo >= e_hi) {
    if (tid == 0) *count = 0u;
    return;
  }
  const size_t slot0 = static_cast<size_t>(head) * p.t_cap;
  const uint32_t cut_k = random_cut(n_sel, n_cand);
  // positions through a buffer resource ending at e_hi (a slot past it reads 0 without a memory
  // access), so no load waits behind a branch
  const __amdgpu_buffer_rsrc_t rp = rsrc_of(p.pos ? p.pos + slot0 : p.seq_len, p.pos ? e_hi * 4 : 0);
  const uint32_t c1 = p.shared_draw ? 0u : (static_cast<uint32_t>(l + p.layer_base) << 16) | static_cast<uint32_t>(h);
  // the chunk's candidates: wave w holds slots c_lo + w*64*R + 64i + lane in round i
  const int jb = c_lo + wave * 64 * R + lane;
  uint32_t key[R];
  bool pass[R];
  constexpr int GR = R % 4 == 0 ? 4 : 1;   // rounds per group of draws
#pragma unroll
  for (int g = 0; g < R; g += GR) {
    uint32_t c0s[GR], w[GR];
#pragma unroll
    for (int k = 0; k < GR; ++k) {
      const int j = jb + (g + k) * 64;
      c0s[k] = p.pos ? ld32(rp, j * 4, 0) : static_cast<uint32_t>(j);
    }
    philox_group<GR>(w, c0s, lane, c1, static_cast<uint32_t>(s), p.event, p.seed_lo, p.seed_hi);
#pragma unroll
    for (int k = 0; k < GR; ++k) {
      key[g + k] = w[k];
      pass[g + k] = jb + (g + k) * 64 < e_hi && w[k] >= cut_k;
    }
  }
  uint32_t c = 0u;
#pragma unroll
  for (int i = 0; i < R; ++i) c += static_cast<uint32_t>(__popcll(__ballot(pass[i])));
  if (lane == 0) cnt[wave] = c;
  __syncthreads();
  uint32_t base = 0u, total = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w < wave) base += cnt[w];
    total += cnt[w];
  }
  uint32_t *lst = p.split_list + (static_cast<size_t>(head) * p.split_chunks + chunk) * (2 * kSplitChunk);
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const uint64_t b = __ballot(pass[i]);
    if (pass[i]) {
      const uint32_t at = base + lanes_below(b);
      lst[2 * at] = key[i];
      lst[2 * at + 1] = static_cast<uint32_t>(jb + i * 64);
    }
    base += static_cast<uint32_t>(__popcll(b));
  }
  if (tid == 0) *count = total;
}

// The ranking workgroup's side of the split draw: gather the head's chunk lists into LDS (chunk
// order is slot order), then the threshold and the placement over the list. False, with the shared
// state to be reset by the caller's full path, when the lists do not fit or cannot be ranked.
template <int NT>
__device__ __forceinline__ bool split_rank(const SelectParams &p, const SelectSmem &sm, const SelectHead &hd) {
  const int tid = threadIdx.x;
  const int C = p.split_chunks;   // at most kSplitMaxChunks = NT / 64 (one count per wave slot)
  for (int i = tid; i < kValueBins; i += NT) {
    sm.hist[i] = 0u;
    sm.mlist[i] = 0u;
  }
  if (tid == 0) *sm.n_members = 0u;
  if (tid < C) sm.cnt_l[tid] = p.split_count[static_cast<size_t>(hd.head) * C + tid];
  __syncthreads();
  uint32_t total = 0u;
  for (int c = 0; c < C; ++c) total += sm.cnt_l[c];
  const uint32_t p_sel = static_cast<uint32_t>(hd.n_sel);
  if (total < p_sel || total > static_cast<uint32_t>(sm.list_cap)) return false;
  // list entry g lies in chunk c with pre[c] <= g < pre[c + 1]; every thread issues its loads
  // before writing any of them to LDS
  constexpr int GPT = (kListMax + NT - 1) / NT;   // list entries per thread at most
  uint32_t pre[kSplitMaxChunks];
  {
    uint32_t acc = 0u;
#pragma unroll
    for (int c = 0; c < kSplitMaxChunks; ++c) {
      pre[c] = acc;
      if (c < C) acc += sm.cnt_l[c];
    }
  }
  uint2 got[GPT];
#pragma unroll
  for (int q = 0; q < GPT; ++q) {
    const uint32_t g = static_cast<uint32_t>(tid + q * NT);
    got[q] = make_uint2(0u, 0u);
    if (g < total) {   // whole waves past the list skip their entry
      int c = 0;
#pragma unroll
      for (int k = 1; k < kSplitMaxChunks; ++k)
        if (k < C && pre[k] <= g) c = k;
      const uint32_t e = g - pre[c];
      got[q] = reinterpret_cast<const uint2 *>(p.split_list + (static_cast<size_t>(hd.head) * C + c) * (2 * kSplitChunk))[e];
    }
  }
#pragma unroll
  for (int q = 0; q < GPT; ++q) {
    const uint32_t g = static_cast<uint32_t>(tid + q * NT);
    if (g < total) {
      sm.lkey[g] = got[q].x;
      sm.lslot[g] = got[q].y;
    }
  }
  __syncthreads();
  uint32_t thr = 0u, need = 0u;
  bool all_ties = true;
  if (!list_threshold<NT, true>(sm, total, p_sel, 0.f, 0.f, random_cut(hd.n_sel, hd.n_cand), thr, need, all_ties))
    return false;
  list_place<NT, true>(sm, total, thr, need, all_ties, hd.P, hd.out, p.b_cap);
  return true;
}

// One workgroup per (layer, seq, KV head): the partition, the fixed places of the prompt and the
// recent window, then the ranking over R rounds, R the smallest of KPT/4, KPT/2 and KPT whose
// NT*R slots reach the last evictable one.
template <int NT, int KPT, int KIND>
__global__ __launch_bounds__(NT) void select_kernel(const SelectParams p) {
  constexpr int NW = NT / 64;
  __shared__ __align__(16) uint32_t hist[kValueBins];
  __shared__ float fred[2 * NW];
  __shared__ uint32_t red[2 * NW];
  __shared__ uint32_t cnt_a[NW];
  __shared__ uint32_t cnt_e[NW];
  __shared__ uint32_t found[3];
  __shared__ uint32_t n_members;
  __shared__ uint32_t shist[kSampleBins];
  __shared__ __align__(16) uint32_t mlist[kValueBins];
  __shared__ uint32_t cnt_l[NW];
  __shared__ uint32_t lkey[list_cap<NT, KPT>()];
  __shared__ uint32_t lslot[list_cap<NT, KPT>()];
  SelectSmem sm;   // filled field by field: an aggregate initialiser of LDS addresses is not
                   // accepted by the unoptimised device build
  sm.hist = hist;
  sm.fred = fred;
  sm.red = red;
  sm.cnt_a = cnt_a;
  sm.cnt_e = cnt_e;
  sm.found = found;
  sm.n_members = &n_members;
  sm.shist = shist;
  sm.mlist = mlist;
  sm.cnt_l = cnt_l;
  sm.lkey = lkey;
  sm.lslot = lslot;
  sm.list_cap = list_cap<NT, KPT>();

  const int tid = threadIdx.x;
  SelectHead hd;
  hd.head = blockIdx.x;
  hd.h = hd.head % p.H;
  hd.s = (hd.head / p.H) % p.S;
  hd.l = hd.head / (p.H * p.S);
  // per-sequence values are uniform: keep them in scalar registers
  const int T = __builtin_amdgcn_readfirstlane(min(max(p.seq_len[hd.s], 0), p.t_cap));
  const int P = __builtin_amdgcn_readfirstlane(min(max(p.prompt_len[hd.s], 0), min(p.prompt_cap, T)));
  const int B = p.budget;
  int32_t *out = p.kept + static_cast<size_t>(hd.head) * p.b_cap;
  const bool writer = (hd.l == 0 && hd.h == 0 && tid == 0);

  if (T <= B) {  // nothing to compress: keep 0..T-1
    for (int r = tid; r < p.b_cap; r += NT) out[r] = r < T ? r : -1;
    if (writer) p.n_kept[hd.s] = T;
    return;
  }
  const int Rw = min(p.recent, min(max(0, B - P), T - P));
  hd.P = P;
  hd.e_lo = P;
  hd.e_hi = T - Rw;
  hd.n_sel = max(0, B - P - Rw);
  hd.n_cand = hd.e_hi - hd.e_lo;
  hd.out = out;
  const int n_kept = max(B, P);
  for (int r = tid; r < P; r += NT) out[r] = r;
  for (int r = tid; r < Rw; r += NT) out[P + hd.n_sel + r] = hd.e_hi + r;
  for (int r = n_kept + tid; r < p.b_cap; r += NT) out[r] = -1;
  if (writer) p.n_kept[hd.s] = n_kept;
  if (hd.n_sel <= 0) return;   // n_sel > 0 implies n_cand > n_sel (T > B)

  // the split draw's ranking side (its chunk workgroups ran just before; only random selection on
  // the 1024-thread tiers is launched with them, whose 16 waves hold the chunk counts)
  if (NT == 1024 && KIND == 1 && p.split_chunks > 0 && listable(hd.n_sel, hd.n_cand, list_cap<NT, KPT>())) {
    if (split_rank<NT>(p, sm, hd)) return;
    __syncthreads();   // every thread has read the shared state before the full path resets it
  }

  const int rounds = (hd.e_hi + NT - 1) / NT;
  if (KPT >= 8 && rounds <= KPT / 4) select_rounds<NT, (KPT >= 8 ? KPT / 4 : KPT), KIND>(p, sm, hd);
  else if (KPT >= 4 && rounds <= KPT / 2) select_rounds<NT, (KPT >= 4 ? KPT / 2 : KPT), KIND>(p, sm, hd);
  else select_rounds<NT, KPT, KIND>(p, sm, hd);
}

// The re-reading kernel: caches past the register tiers (past 32768 slots; context lengths reach
// 128K tokens), and random selection from 16385 slots on (no keys held in registers, so its
// workgroups share CUs with a concurrent kernel). The same rankings, threshold rule and ordered
// scan as the register kernel, with every step recomputing the keys from memory (a score load, or
// the Philox draw). Top-k and random first take the listed path (a cut, one sweep that lists the
// keys at or above it in LDS, the threshold and placement over the list; random selections of more
// than half list the words to evict, complemented, and place by the ordered scan); the fallback steps are
// min/max (scores) and the 1024-bin histogram, the threshold bin's keys ranked in LDS (or, when
// crowded, OR/AND and 8-bit radix passes), then the ordered scan in chunks of 4 * NT slots in slot
// order with the kept and tied counts carried from chunk to chunk. The union (KIND 2) runs G + 1
// such passes and keeps its union as a bit per slot in dynamic LDS (t_cap / 8 bytes); a listed
// head pass marks its selected slots from the list.
constexpr int kStreamThreads = 1024;
constexpr int kLeanRandomThreads = 512;   // random selection within the register tiers' sizes
static_assert(kSelectMaxSlotsUnion / 8 <= 32 * 1024, "union bits fit in 32 KB of LDS");

template <int KIND, int NT = kStreamThreads>
__global__ __launch_bounds__(NT) void select_stream_kernel(const SelectParams p) {
  constexpr int NW = NT / 64;
  constexpr bool RANDOM = KIND == 1, UNION = KIND == 2;
  __shared__ __align__(16) uint32_t hist[kValueBins];
  __shared__ uint32_t red[2 * NW];
  __shared__ uint32_t wsum[2 * NW];
  __shared__ uint32_t found[3];
  __shared__ uint32_t n_members;
  __shared__ uint32_t kb[2];   // key interval of the threshold's bin
  extern __shared__ uint32_t ubits[];   // union: bit j set when slot j is in some head's top-k
  // the listed path: keys and slots of the candidates at or above the cut
  constexpr int LCAP = kListMax;
  __shared__ uint32_t lkey[LCAP];
  __shared__ uint32_t lslot[LCAP];
  __shared__ __align__(16) uint32_t mlist[kValueBins];
  __shared__ uint32_t shist[kSampleBins];

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
  const uint32_t c1 = p.shared_draw ? 0u : (static_cast<uint32_t>(l + p.layer_base) << 16) | static_cast<uint32_t>(h);
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
    // The row (scores) or the positions (random) are read through buffer resources over [0, e_hi):
    // a read past e_hi returns 0 without a memory access, so the sweeps below issue their loads
    // unconditionally (a load under a per-slot condition waits for everything in flight).
    const __amdgpu_buffer_rsrc_t rrow = rsrc_of(RANDOM ? static_cast<const void *>(p.seq_len) : row,
                                                RANDOM ? 0 : e_hi * 4);
    const __amdgpu_buffer_rsrc_t rpos = rsrc_of(p.pos ? static_cast<const void *>(p.pos + slot0) : p.seq_len,
                                                p.pos ? e_hi * 4 : 0);
    // the key of slot j from the 4 bytes loaded for it (a score's bits, or a position)
    auto key_from = [&](int j, uint32_t bits) -> uint32_t {
      if (RANDOM) {
        const uint32_t c0 = p.pos ? bits : static_cast<uint32_t>(j);
        return philox_draw(c0, c1, static_cast<uint32_t>(s), p.event, p.seed_lo, p.seed_hi);
      }
      const uint32_t k = order_key(__uint_as_float(bits));
      if (UNION && last) {
        const bool in_u = in_union(j);
        if (long_union && !in_u) return 0u;
        if (!long_union && in_u) return 0xFFFFFFFFu;
      }
      return k;
    };
    auto load_of = [&](int j) -> uint32_t {
      if (RANDOM) return p.pos ? ld32(rpos, j * 4, 0) : 0u;
      return ld32(rrow, j * 4, 0);
    };
    // visit(j, key) for every candidate slot, U loads in flight per thread (fewer for the draw,
    // whose keys cost far more arithmetic than their position loads)
    auto sweep = [&](auto &&visit) __attribute__((always_inline)) {
      constexpr int U = RANDOM ? 2 : 8;
      for (int j = e_lo + tid; j < e_hi; j += U * NT) {
        uint32_t b[U];
#pragma unroll
        for (int u = 0; u < U; ++u) b[u] = load_of(j + u * NT);
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (j + u * NT < e_hi) visit(j + u * NT, key_from(j + u * NT, b[u]));
      }
    };
    const int p_sel = UNION && !last ? k_head : n_sel;

    // mode: 0 = select none, 1 = select all candidates, 2 = threshold rule
    int mode;
    uint32_t thr = 0u, need = 0u;
    bool all_ties = false;  // every key equal to thr is taken
    bool listed = false;    // the threshold came from the list, which is still in LDS
    uint32_t n_list = 0u;
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
      float scale = 0.f, off = 0.f, fmin = 0.f, fmax = 0.f;
      auto bin_of = [&](uint32_t k) { return RANDOM ? (k >> 22) : bin_of_key(k, scale, off); };
      {   // the listed path's LDS starts cleared (ordered before use by the barriers below)
        for (int i = tid; i < kValueBins; i += NT) mlist[i] = 0u;
        for (int i = tid; i < kSampleBins; i += NT) shist[i] = 0u;
        for (int i = tid; i < kValueBins; i += NT) hist[i] = 0u;
        if (tid == 0) n_members = 0u;
      }
      if (!RANDOM) {
        uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
        sweep([&](int, uint32_t k) {
          if (k > kKeyNegInf && k < kKeyPosInf) {
            kmn = min(kmn, k);
            kmx = max(kmx, k);
          }
        });
        block_min_max<NT>(kmn, kmx, red);
        fmin = key_value(kmn);
        fmax = key_value(kmx);
        scale = static_cast<float>(kValueBins) / (fmax - fmin);
        off = -fmin * scale;
        binned = kmn < kmx && scale > 0.f && scale < 3.0e38f && fabsf(off) < 3.0e38f;
      }

      // ---- listed path: a cut from a strided sample (scores) or the selection's share (random
      // words); one sweep counts the candidates at or above it and lists them in LDS in slot order
      // (chunks of 4 * NT slots, a block-wide scan each); the threshold is then found on the list
      // as in the register kernel. A cut that leaves fewer than p_sel or more than the list holds,
      // or a crowded threshold bin, falls back to the sweeps below.
      // the want_n largest keys, or with fl (random words only) the want_n lowest, listed complemented
      auto flipped_key = [&](uint32_t k) { return ~k; };
      auto stream_list = [&](int want_n, bool fl) -> bool {
        uint32_t cut = 1u;   // list keys >= cut (order keys, or words)
        float lo_f = fmin;
        if (RANDOM) {
          const float want = static_cast<float>(want_n) + 4.f * sqrtf(static_cast<float>(want_n)) + 16.f;
          if (want < static_cast<float>(n_cand)) {
            const double c = 4294967296.0 * (1.0 - static_cast<double>(want) / static_cast<double>(n_cand));
            cut = c > 1.0 ? static_cast<uint32_t>(c) : 1u;
          }
        } else {
          // the sample: 128 blocks of 32 consecutive candidates (one 128-byte line each) spread
          // evenly over the evictable range. Single keys at a stride would fetch a line apiece;
          // fewer, longer blocks miss top keys bunched between them (scores rising with the slot).
          const float sscale = static_cast<float>(kSampleBins) / (fmax - fmin), soff = -fmin * sscale;
          constexpr int kBlock = 32, kBlocks = kStreamSamples / kBlock, SPT = kStreamSamples / NT;
          static_assert(kStreamSamples % NT == 0, "whole sample rounds per thread");
          const int step = max(kBlock, n_cand / kBlocks);
          uint32_t sb[SPT];
#pragma unroll
          for (int u = 0; u < SPT; ++u) {
            const int i = tid + u * NT;
            sb[u] = load_of(e_lo + (i / kBlock) * step + (i % kBlock));
          }
#pragma unroll
          for (int u = 0; u < SPT; ++u) {
            const int i = tid + u * NT;
            const int off = (i / kBlock) * step + (i % kBlock);
            if (off < n_cand)
              atomicAdd(&shist[bin_of_key_n(key_from(e_lo + off, sb[u]), sscale, soff, kSampleBins)], 1u);
          }
          __syncthreads();
          uint32_t bc, above_s, n_s;
          wave_find_bin<kSampleBins>(shist, [&](uint32_t tot) {
            const float lam = static_cast<float>(want_n) * static_cast<float>(tot) / static_cast<float>(n_cand);
            return static_cast<uint32_t>(lam + 3.f * sqrtf(lam) + 4.f);
          }, lane, bc, above_s, n_s);
          cut = 0u;
          if (bc > 1u) {
            lo_f = (static_cast<float>(bc - 1u) - soff) / sscale;
            cut = order_key(lo_f);
          }
        }
        // KC consecutive candidates per thread and chunk, the next chunk's loads issued before
        // this chunk's keys are formed and listed (the last chunk's next reads past e_hi: no access).
        // Random draws at the slots' own positions start their chunks at a multiple of 4 slots, so
        // a thread's 8 slots are exactly two Philox blocks (slots below e_lo take no part).
        constexpr int KC = RANDOM ? 8 : 4;
        const bool blocks = RANDOM && !p.pos;
        const int c_first = blocks ? (e_lo & ~3) : e_lo;
        uint32_t nxt[KC];
#pragma unroll
        for (int q = 0; q < KC; ++q) nxt[q] = load_of(c_first + KC * tid + q);
        uint32_t carry = 0u;
        for (int c = c_first; c < e_hi; c += KC * NT) {
          const int j0 = c + KC * tid;
          uint32_t cur[KC];
#pragma unroll
          for (int q = 0; q < KC; ++q) {
            cur[q] = nxt[q];
            nxt[q] = load_of(j0 + KC * NT + q);
          }
          uint32_t kk[KC];
          uint32_t f = 0u;
          if (RANDOM && blocks) {
            uint32_t w8[8];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
              const uint4 blk = philox_block(static_cast<uint32_t>(j0 >> 2) + b, c1, static_cast<uint32_t>(s), p.event,
                                             p.seed_lo, p.seed_hi);
              w8[4 * b] = blk.x;
              w8[4 * b + 1] = blk.y;
              w8[4 * b + 2] = blk.z;
              w8[4 * b + 3] = blk.w;
            }
#pragma unroll
            for (int q = 0; q < KC; ++q) {
              kk[q] = 0u;
              if (j0 + q >= e_lo && j0 + q < e_hi) {
                kk[q] = fl ? flipped_key(w8[q]) : w8[q];
                f |= static_cast<uint32_t>(kk[q] >= cut) << q;
              }
            }
          } else {
#pragma unroll
            for (int q = 0; q < KC; ++q) {
              kk[q] = 0u;
              if (j0 + q < e_hi) {
                kk[q] = key_from(j0 + q, cur[q]);
                if (RANDOM && fl) kk[q] = flipped_key(kk[q]);
                f |= static_cast<uint32_t>(kk[q] >= cut) << q;
              }
            }
          }
          const uint32_t cnt = static_cast<uint32_t>(__popc(f));
          const uint32_t x = wave_inclusive_sum(cnt);
          if (lane == 63) wsum[wave] = x;
          __syncthreads();
          uint32_t at = carry + x - cnt, tot = 0u;
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            if (w < wave) at += wsum[w];
            tot += wsum[w];
          }
          __syncthreads();   // wsum is rewritten by the next chunk
#pragma unroll
          for (int q = 0; q < KC; ++q) {
            if ((f >> q) & 1u) {
              if (at < static_cast<uint32_t>(LCAP)) {
                lkey[at] = kk[q];
                lslot[at] = static_cast<uint32_t>(j0 + q);
              }
              ++at;
            }
          }
          carry += tot;
        }
        __syncthreads();   // the last chunk's list entries are written before anyone reads the list
        if (carry < static_cast<uint32_t>(want_n) || carry > static_cast<uint32_t>(LCAP)) return false;
        const float scale2 = static_cast<float>(kListBins) / (fmax - lo_f), off2 = -lo_f * scale2;
        if (!RANDOM && !(fmax > lo_f && scale2 > 0.f && scale2 < 3.0e38f && fabsf(off2) < 3.0e38f)) return false;
        const uint32_t span = 0xFFFFFFFFu - cut;
        const int bits = span ? 32 - __clz(span) : 0;
        const int shift = bits > 8 ? bits - 8 : 0;
        auto lbin = [&](uint32_t k) {
          return RANDOM ? (k - cut) >> shift : bin_of_key_n(k, scale2, off2, kListBins);
        };
        for (uint32_t e = tid; e < carry; e += NT) atomicAdd(&hist[lbin(lkey[e])], 1u);
        __syncthreads();
        uint32_t b, above, tot;
        wave_find_bin<kListBins>(hist, [&](uint32_t) { return static_cast<uint32_t>(want_n); }, lane, b, above, tot);
        const uint32_t rem = static_cast<uint32_t>(want_n) - above;
        for (uint32_t e = tid; e < carry; e += NT) {
          const uint32_t k = lkey[e];
          if (lbin(k) == b) {
            const uint32_t at = atomicAdd(&n_members, 1u);
            if (at < member_cap<NT>()) mlist[at] = k;
          }
        }
        __syncthreads();
        const uint32_t m = n_members;
        if (m > member_cap<NT>()) return false;
        rank_members<NT>(mlist, m, rem, found);   // entries past m are still zero
        __syncthreads();
        thr = found[0];
        need = found[1];
        all_ties = found[2] == need;
        n_list = carry;
        return true;
      };
      // Random, more than half selected: the q = n_cand - p_sel words to evict listed complemented
      // (as in the register kernel), then the ordered scan below places the kept set; one draw
      // fewer per key than the fallback's sweeps. For scores the same listing and scan measured
      // slower than the fallback (0.53-0.56 against 0.46-0.47 ms on 576 heads of 131,072 slots
      // with 4,000 to evict), so scores keep it.
      bool flipped = false;
      const int q_evict = n_cand - p_sel;
      const bool list_top = (RANDOM || binned) && 2 * p_sel <= n_cand && p_sel + p_sel / 8 + 64 <= LCAP;
      const bool list_low = RANDOM && !list_top && 2 * q_evict <= n_cand && q_evict + q_evict / 8 + 64 <= LCAP;
      if (list_top || list_low) {   // one call site: the listing is inlined once
        const bool ok = stream_list(list_low ? q_evict : p_sel, list_low);
        listed = list_top && ok;
        flipped = list_low && ok;
        if (flipped) {
          const uint32_t ties_at = found[2];   // words equal to the q-th lowest
          thr = ~thr;
          need = ties_at - need;               // the ties kept: those the q lowest leave
          all_ties = need == ties_at;
        }
      }
      if (!listed && !flipped) {
      __syncthreads();   // the listed path's readers of hist are done
      if (binned) {
        for (int i = tid; i < kValueBins; i += NT) hist[i] = 0u;
        if (tid == 0) n_members = 0u;
        __syncthreads();
        sweep([&](int, uint32_t k) { atomicAdd(&hist[bin_of(k)], 1u); });
        __syncthreads();
        if (wave == 0) find_bin<kValueBins>(hist, remaining, lane, found);
        __syncthreads();
        bsel = found[0];
        remaining -= found[1];
        bin_interval<RANDOM>(bsel, scale, off, wave, lane, kb);
        __syncthreads();  // `found` and `hist` are reused below; kb is written
        klo = kb[0];
        khi = kb[1];
        // a short member list is ranked directly (as in the register kernel)
        sweep([&](int, uint32_t k) {
          if (k >= klo && k <= khi) {
            const uint32_t at = atomicAdd(&n_members, 1u);
            if (at < member_cap<NT>()) hist[at] = k;
          }
        });
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
        sweep([&](int, uint32_t k) {
          if (member(k)) {
            kor |= k;
            kand &= k;
          }
        });
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
            sweep([&](int, uint32_t k) {
              if ((k & mask) == prefix && member(k)) atomicAdd(&hist[(k >> lo) & dmask], 1u);
            });
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
    }

    // ---- placement from the list: the pins arithmetically, the selected slots by one block-wide
    // scan over contiguous runs of list entries (as in the register kernel); a union head pass
    // marks its selected slots in the union's bits instead
    if (listed) {
      const bool mark = UNION && !last;
      if (!mark) {
        for (int r = tid; r < P; r += NT) out[r] = r;
        for (int r = tid; r < Rw; r += NT) out[P + n_sel + r] = e_hi + r;
      }
      const uint32_t n = n_list;
      const uint32_t per = (n + NT - 1) / NT;
      const uint32_t e0 = min(n, static_cast<uint32_t>(tid) * per), e1 = min(n, e0 + per);
      auto is_a = [&](uint32_t k) { return all_ties ? k >= thr : k > thr; };
      uint32_t ca = 0u, ct = 0u;
      for (uint32_t e = e0; e < e1; ++e) {
        const uint32_t k = lkey[e];
        ca += is_a(k) ? 1u : 0u;
        ct += (!all_ties && k == thr) ? 1u : 0u;
      }
      const uint32_t packed = ca | (ct << 16);   // both at most kListMax
      const uint32_t incl = wave_inclusive_sum(packed);
      if (lane == 63) wsum[wave] = incl;
      __syncthreads();
      uint32_t below = incl - packed;
      for (int w = 0; w < wave; ++w) below += wsum[w];
      uint32_t ra = below & 0xFFFFu, re = below >> 16;
      for (uint32_t e = e0; e < e1; ++e) {
        const uint32_t k = lkey[e];
        uint32_t o = 0xFFFFFFFFu;
        if (is_a(k)) {
          o = static_cast<uint32_t>(P) + ra + min(re, need);
          ++ra;
        } else if (!all_ties && k == thr) {
          if (re < need) o = static_cast<uint32_t>(P) + ra + re;
          ++re;
        }
        if (mark) {
          if (o != 0xFFFFFFFFu) atomicOr(&ubits[lslot[e] >> 5], 1u << (lslot[e] & 31u));
        } else if (o < static_cast<uint32_t>(p.b_cap)) {
          out[o] = static_cast<int32_t>(lslot[e]);
        }
      }
      if (mark) __syncthreads();   // the union's bits are complete before the next pass reads them
      continue;
    }

    if (UNION && !last && (mode != 2 || all_ties)) {
      // a head's top-k needs no order: mark every candidate above (or at) the threshold
      if (mode == 2) {
        sweep([&](int j, uint32_t k) {
          if (k >= thr) atomicOr(&ubits[j >> 5], 1u << (j & 31));
        });
      } else if (mode == 1) {
        for (int j = e_lo + tid; j < e_hi; j += NT) atomicOr(&ubits[j >> 5], 1u << (j & 31));
      }
      __syncthreads();
      continue;
    }

    // ordered scan: thread t takes slots c + 4t .. c + 4t + 3 of each chunk. The last pass writes
    // the kept list; a union head pass adds its top-k (ties to the lower slots) to the union.
    // The union's passes (which always scan) issue the keys' loads for chunk c + 1 before chunk c
    // is ranked (reads at or past e_hi return 0 without an access; bits loaded for slots below
    // e_lo are not used); top-k and random scan only on their fallback and keep the registers.
    constexpr bool AHEAD = UNION;
    uint32_t carry_a = 0u, carry_e = 0u;  // unconditional / tied slots in earlier chunks
    uint32_t nb4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) nb4[q] = AHEAD && mode == 2 ? load_of(4 * tid + q) : 0u;
    for (int c = 0; c < T; c += 4 * NT) {
      const int j0 = c + 4 * tid;
      uint32_t cb4[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        cb4[q] = nb4[q];
        nb4[q] = AHEAD && mode == 2 ? load_of(j0 + 4 * NT + q) : 0u;
      }
      uint32_t fa = 0u, fe = 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = j0 + q;
        if (j >= T) break;
        const bool cnd = j >= e_lo && j < e_hi;
        bool a = last ? (!cnd || mode == 1) : (cnd && mode == 1), e = false;  // pins: last pass
        if (cnd && mode == 2) {
          const uint32_t k = key_from(j, AHEAD ? cb4[q] : load_of(j));
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
template <int NT, int KPT>
hipError_t launch_cfg(const SelectParams &p, SelectKind kind, dim3 grid, hipStream_t st) {
  if (kind == SelectKind::kUnion)
    hipLaunchKernelGGL((select_kernel<NT, KPT, 2>), grid, dim3(NT), 0, st, p);
  else if (kind == SelectKind::kRandom)
    hipLaunchKernelGGL((select_kernel<NT, KPT, 1>), grid, dim3(NT), 0, st, p);
  else
    hipLaunchKernelGGL((select_kernel<NT, KPT, 0>), grid, dim3(NT), 0, st, p);
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

// The split draw applies to random selection over batches of at most kSplitMaxHeads heads whose
// caches fill the 1024-thread register tiers (one workgroup per head would leave most CUs idle);
// its scratch is a count and a list of kSplitChunk entries per chunk. The selectors share one
// workspace query, so top-k callers size for it too.
#ifndef KV_SPLIT_MAX_HEADS
#define KV_SPLIT_MAX_HEADS 64
#endif
constexpr long long kSplitMaxHeads = KV_SPLIT_MAX_HEADS;
static bool split_shape(long long heads, int t_cap) {
  return heads <= kSplitMaxHeads && t_cap > 8192 && t_cap <= kSelectMaxSlots;
}
static size_t split_count_bytes(long long heads, int chunks) {
  return (static_cast<size_t>(heads) * chunks * 4 + 255) & ~static_cast<size_t>(255);
}

size_t select_scratch_bytes(int L, int S, int H, int t_cap) {
  const long long heads = static_cast<long long>(L) * S * H;
  if (!split_shape(heads, t_cap)) return 0;
  const int chunks = (t_cap + kSplitChunk - 1) / kSplitChunk;
  return split_count_bytes(heads, chunks) + static_cast<size_t>(heads) * chunks * kSplitChunk * 8;
}

hipError_t launch_select(const SelectParams &p, SelectKind kind, hipStream_t st) {
  const long long heads = static_cast<long long>(p.L) * p.S * p.H;
  if (heads <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(heads));
  const int t = p.t_cap;
  // Random selection on few heads with long caches: the chunk workgroups draw and list first, then
  // the tier's ranking workgroups.
  // (n_sel never exceeds the budget: a budget whose selection cannot fit the list rules it out)
  const int split_cap = t <= 1024 * 16 ? list_cap<1024, 16>() : list_cap<1024, 32>();
  if (kind == SelectKind::kRandom && p.scratch && split_shape(heads, t) &&
      static_cast<long long>(p.budget) + p.budget / 8 + 64 <= split_cap) {
    SelectParams q = p;
    q.split_chunks = (t + kSplitChunk - 1) / kSplitChunk;
    q.split_list_cap = split_cap;
    q.split_count = static_cast<uint32_t *>(p.scratch);
    q.split_list = reinterpret_cast<uint32_t *>(static_cast<char *>(p.scratch) + split_count_bytes(heads, q.split_chunks));
    const dim3 sgrid(static_cast<unsigned>(heads * q.split_chunks));
    hipLaunchKernelGGL(select_split_kernel, sgrid, dim3(kSplitThreads), 0, st, q);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return t <= 1024 * 16 ? launch_cfg<1024, 16>(q, kind, grid, st) : launch_cfg<1024, 32>(q, kind, grid, st);
  }
  // Random selection over 16,385-32,768 slots: the re-reading kernel at 512 threads, which draws
  // each key once on its listed path and holds no keys in registers (50 VGPRs against the
  // 1024 x 32 tier's 119). Two of its workgroups share a CU, and beside another kernel (the
  // compaction of a previous layer chunk) they find room on CUs that the tier's, which need a
  // whole CU's registers, do not. On 2,304 heads it draws in 0.157 ms against 0.186 ms; on 256
  // heads or fewer (one workgroup per CU) it takes about 15 % longer than 1,024 threads would.
  // A budget over half the cache (periodic eviction of a small buffer) stays in the register tier:
  // there a selection of more than half the candidates lists the keys to evict, where the
  // re-reading kernel would redraw every key in each of its fallback sweeps.
  if (kind == SelectKind::kRandom && t > 1024 * 16 && t <= kSelectMaxSlots && 2ll * p.budget <= t) {
    hipLaunchKernelGGL((select_stream_kernel<1, kLeanRandomThreads>), grid, dim3(kLeanRandomThreads), 0, st, p);
    return hipGetLastError();
  }
  // Register tiers: NT threads x KPT rounds of one key each cover t_cap slots.
  if (t <= kSelectMaxSlots) {
    if (t <= 256 * 8) return launch_cfg<256, 8>(p, kind, grid, st);
    if (t <= 256 * 16) return launch_cfg<256, 16>(p, kind, grid, st);
    if (t <= 512 * 16) return launch_cfg<512, 16>(p, kind, grid, st);
    if (t <= 1024 * 16) return launch_cfg<1024, 16>(p, kind, grid, st);
    return launch_cfg<1024, 32>(p, kind, grid, st);
  }
  // Past the tiers, the re-reading kernel (the union keeps its bits in dynamic LDS).
  if (kind == SelectKind::kUnion) {
    if (t > kSelectMaxSlotsUnion) return hipErrorInvalidValue;
    const size_t union_bytes = static_cast<size_t>((t + 31) / 32) * 4;
    hipLaunchKernelGGL(select_stream_kernel<2>, grid, dim3(kStreamThreads), union_bytes, st, p);
  } else if (kind == SelectKind::kRandom) {
    hipLaunchKernelGGL(select_stream_kernel<1>, grid, dim3(kStreamThreads), 0, st, p);
  } else {
    hipLaunchKernelGGL(select_stream_kernel<0>, grid, dim3(kStreamThreads), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace kvevict

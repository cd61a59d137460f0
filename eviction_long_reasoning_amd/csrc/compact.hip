// Gather-compaction of kept K/V rows for gfx950.
//
// What is computed: "Random Attention: Rethinking KV Cache Eviction for
// Efficient Reasoning", Appendix F ("Engine details"): after each eviction
// the KV tensors are compacted with a gather, keep-sets in chronological
// order. Row r of a head's output is row kept[r] of its input, for K, V and
// the positions.
//
// Mapping: a row of d elements is row16 16-byte pieces; G = row16 rounded up to a power of two
// lanes copy one row (16-byte loads and stores), 256/G rows per pass. Workgroups come in pairs
// over the same output rows of one head, the even one moving K (and the positions), the odd one
// V, two passes each; every thread keeps one row piece in flight and loads the next pass's kept
// index before the current pass's row, so the index is not on the row's path. Stores are fully
// contiguous and loads are whole rows (kept indices ascend, so neighbouring kept rows often share
// DRAM pages).
//
// Hole filling is the in-place alternative: only kept rows at or beyond the
// new length move, each into an evicted slot below it, so a periodic eviction
// that drops a few hundred rows per head moves a few hundred rows instead of
// rewriting the whole cache. Slot order then stops being chronological and the
// positions move with the rows.
#include "kv_internal.hpp"

namespace kvevict {
namespace {

constexpr int kCompactThreads = 256;
constexpr int kPasses = 2;   // passes of 256 / G rows per workgroup

// Every row is moved exactly once, so loads and stores use the non-temporal cache policy.
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const uint4 *p) {
  const v4u32 v = __builtin_nontemporal_load(reinterpret_cast<const v4u32 *>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st_stream(uint4 *p, const uint4 &x) {
  const v4u32 v = {x.x, x.y, x.z, x.w};
  __builtin_nontemporal_store(v, reinterpret_cast<v4u32 *>(p));
}

template <int G>
__global__ __launch_bounds__(kCompactThreads) void compact_kernel(const CompactParams p) {
  constexpr int ROWS_PER_PASS = kCompactThreads / G;
  const int wg = static_cast<int>(blockIdx.x >> 1);
  const int which = static_cast<int>(blockIdx.x & 1);   // 0: K and the positions, 1: V
  const int head = wg / p.wgs_per_head;
  const int part = wg - head * p.wgs_per_head;
  const int s = (head / p.H) % p.S;
  const int nk = min(min(max(p.n_kept[s], 0), p.b_cap), p.out_cap);
  const int r0 = part * ROWS_PER_PASS * kPasses;
  if (r0 >= nk) return;

  const int c = threadIdx.x % G;
  const int rr = threadIdx.x / G;
  const bool lane_live = c < p.row16;
  const size_t in_row0 = static_cast<size_t>(head) * p.t_cap;
  const size_t out_row0 = static_cast<size_t>(head) * p.out_cap;
  const int32_t *kept = p.kept + static_cast<size_t>(head) * p.b_cap;
  const uint4 *src = which ? p.V_in : p.K_in;
  uint4 *dst = which ? p.V_out : p.K_out;
  auto source_row = [&](int r) {   // kept[r], or -1 past n_kept or out of range
    const int j = r < nk ? kept[r] : -1;
    return (j >= 0 && j < p.t_cap) ? j : -1;
  };

  int j_next = source_row(r0 + rr);
#pragma unroll
  for (int b = 0; b < kPasses; ++b) {
    const int r = r0 + b * ROWS_PER_PASS + rr;
    const int j = j_next;
    if (b + 1 < kPasses) j_next = source_row(r + ROWS_PER_PASS);
    const bool ld = j >= 0 && lane_live;
    const size_t off = (in_row0 + static_cast<size_t>(ld ? j : 0)) * p.row16 + (ld ? c : 0);
    const uint4 v = ld ? ld_stream(src + off) : make_uint4(0u, 0u, 0u, 0u);
    if (ld) st_stream(dst + (out_row0 + static_cast<size_t>(r)) * p.row16 + c, v);
    if (j >= 0 && c == 0 && which == 0 && p.pos_out)
      p.pos_out[out_row0 + r] = p.pos_in ? p.pos_in[in_row0 + j] : j;
  }
}

// In-place hole filling. With n = n_kept and kept ascending, the kept slots below n are the
// prefix kept[0..r0) and the movers are the suffix kept[r0..n); the holes are the n - r0 slots
// below n missing from the prefix. The i-th hole is i + #{r < r0 : kept[r] - r <= i} (kept[r] - r
// counts the holes before kept[r] and never decreases). Movers are read only from slots >= n and
// written only to slots < n, so no slot is both read and written.
// Kept lists up to this long are copied to LDS first, so that the binary searches (about a dozen
// dependent reads per mover) run at LDS rather than global-memory latency.
constexpr int kHoleStage = 4096;

template <int G>
__global__ __launch_bounds__(kCompactThreads) void holes_kernel(const HoleParams p) {
  constexpr int ROWS_PER_PASS = kCompactThreads / G;
  __shared__ int prefix;
  __shared__ int32_t staged_kept[kHoleStage];
  const int head = blockIdx.x / p.wgs_per_head;
  const int part = blockIdx.x - head * p.wgs_per_head;
  const int s = (head / p.H) % p.S;
  const int n = min(min(max(p.n_kept[s], 0), p.b_cap), p.t_cap);
  const int32_t *kept_g = p.kept + static_cast<size_t>(head) * p.b_cap;
  const bool staged = n <= kHoleStage;
  if (staged)
    for (int r = threadIdx.x; r < n; r += kCompactThreads) staged_kept[r] = kept_g[r];
  __syncthreads();
  auto kept = [&](int r) { return staged ? staged_kept[r] : kept_g[r]; };
  if (threadIdx.x == 0) {
    int lo = 0, hi = n;  // first r with kept[r] >= n
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (kept(mid) < n) lo = mid + 1; else hi = mid;
    }
    prefix = lo;
  }
  __syncthreads();
  const int r0 = prefix;
  const int movers = n - r0;
  const int c = threadIdx.x % G;
  const int rr = threadIdx.x / G;
  const size_t row0 = static_cast<size_t>(head) * p.t_cap;
  for (int i = part * ROWS_PER_PASS + rr; i < movers; i += ROWS_PER_PASS * p.wgs_per_head) {
    const int src = kept(r0 + i);
    if (src < n || src >= p.t_cap) continue;   // not a mover (kept not ascending) or out of range
    int lo = 0, hi = r0;                        // #{r < r0 : kept[r] - r <= i}
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (kept(mid) - mid <= i) lo = mid + 1; else hi = mid;
    }
    const int dst = i + lo;                     // < n
    if (c < p.row16) {
      const size_t so = (row0 + src) * p.row16 + c, dso = (row0 + dst) * p.row16 + c;
      const uint4 k = ld_stream(p.K + so), v = ld_stream(p.V + so);
      st_stream(p.K + dso, k);
      st_stream(p.V + dso, v);
    }
    if (c == 0 && p.pos) p.pos[row0 + dst] = p.pos[row0 + src];
  }
}

}  // namespace

int compact_rows_per_wg(int group) { return (kCompactThreads / group) * kPasses; }
int compact_wgs_per_slice() { return 2; }

hipError_t launch_compact(const CompactParams &p, hipStream_t st) {
  int G = 1;
  while (G < p.row16) G <<= 1;
  if (G > 64) return hipErrorInvalidValue;
  const long long blocks = static_cast<long long>(p.L) * p.S * p.H * p.wgs_per_head * compact_wgs_per_slice();
  if (blocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(blocks)), blk(kCompactThreads);
  switch (G) {
    case 1: hipLaunchKernelGGL(compact_kernel<1>, grid, blk, 0, st, p); break;
    case 2: hipLaunchKernelGGL(compact_kernel<2>, grid, blk, 0, st, p); break;
    case 4: hipLaunchKernelGGL(compact_kernel<4>, grid, blk, 0, st, p); break;
    case 8: hipLaunchKernelGGL(compact_kernel<8>, grid, blk, 0, st, p); break;
    case 16: hipLaunchKernelGGL(compact_kernel<16>, grid, blk, 0, st, p); break;
    case 32: hipLaunchKernelGGL(compact_kernel<32>, grid, blk, 0, st, p); break;
    case 64: hipLaunchKernelGGL(compact_kernel<64>, grid, blk, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_compact_holes(const HoleParams &p, hipStream_t st) {
  int G = 1;
  while (G < p.row16) G <<= 1;
  if (G > 64) return hipErrorInvalidValue;
  const long long blocks = static_cast<long long>(p.L) * p.S * p.H * p.wgs_per_head;
  if (blocks <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(blocks)), blk(kCompactThreads);
  switch (G) {
    case 1: hipLaunchKernelGGL(holes_kernel<1>, grid, blk, 0, st, p); break;
    case 2: hipLaunchKernelGGL(holes_kernel<2>, grid, blk, 0, st, p); break;
    case 4: hipLaunchKernelGGL(holes_kernel<4>, grid, blk, 0, st, p); break;
    case 8: hipLaunchKernelGGL(holes_kernel<8>, grid, blk, 0, st, p); break;
    case 16: hipLaunchKernelGGL(holes_kernel<16>, grid, blk, 0, st, p); break;
    case 32: hipLaunchKernelGGL(holes_kernel<32>, grid, blk, 0, st, p); break;
    case 64: hipLaunchKernelGGL(holes_kernel<64>, grid, blk, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvevict

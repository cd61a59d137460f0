// Addressing of key rows stored after RoPE, shared by the single-centre and the grouped-query
// rotated score kernels. Not part of the public interface.
//
// A wave step reads the KPS consecutive slots jb .. jb + KPS - 1 of one (layer, sequence, KV
// head), jb a multiple of KPS, one slot per group of lanes. In a dense head, or in a paged pool
// whose blocks hold at least KPS slots (blocks start at multiples of their power-of-two size),
// those slots sit at one base address plus a fixed stride per slot, the same for the whole wave.
// Once per 64-slot batch, lane t works out step t's base address and the byte range that ends
// after its last slot below the sequence length (one block-table entry and a few integer
// products per lane); each step then reads its three words back as scalars and hands them to a
// buffer load as its resource. Lanes of slots at or past the sequence length, and lanes given an
// offset beyond every range, read zeros without touching memory. Per step a lane does one load
// at a loop-invariant offset.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvevict {

constexpr int kRowRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kRowLoadNt = 2;              // cache policy "nt": every key row is read once
constexpr int kRowOffIdle = 0x7FFFFFF0;    // lane offset past any step's range: the load returns zeros

// Where the rows of one (layer, sequence, KV head) live. LAYOUT 0: dense [.., t_cap, d] rows from
// `first`; 1: token-major pool [L, n_blocks, block, H, d]; 2: head-major pool [L, n_blocks, H, block, d].
struct RowSpace {
  const char *K;
  int64_t row_bytes;
  int64_t first;    // dense: the head's first row
  int64_t blk0;     // paged: l * n_blocks
  int32_t H, h, shift, n_blocks;
  const int32_t *table;  // paged: this sequence's block-table row
};

// Byte distance between the rows of consecutive slots of one block (or of the dense head).
template <int LAYOUT>
__device__ __forceinline__ int64_t slot_stride(const RowSpace &rs) {
  return LAYOUT == 1 ? rs.H * rs.row_bytes : rs.row_bytes;
}

// Whether every step of this launch can use one base address: always for dense heads; for pools,
// when a block holds a whole step and a step's byte range fits a 32-bit buffer offset.
template <int LAYOUT, int KPS>
__device__ __forceinline__ bool uniform_steps(const RowSpace &rs) {
  if (LAYOUT == 0) return true;
  return (1 << rs.shift) >= KPS && slot_stride<LAYOUT>(rs) * KPS + rs.row_bytes < (int64_t{1} << 30);
}

// Block-table entry of step `lane`'s block in the 64-slot batch starting at j0 (j0 < T): steps at
// or past T take the last block holding a live slot. Entries are taken as stored; batch_steps
// clamps them to the pool.
template <int KPS>
__device__ __forceinline__ int step_entry(const RowSpace &rs, int j0, int T, int lane) {
  const int jb = min(j0 + lane * KPS, T - 1);
  return rs.table[jb >> rs.shift];
}

// Addressing of the steps of one 64-slot batch, computed once per batch with one lane per step:
// lane t holds step t's base address and the byte range ending after its last slot below T.
struct BatchSteps {
  uint32_t lo, hi;
  int32_t range;
};

template <int LAYOUT, int KPS>
__device__ __forceinline__ BatchSteps batch_steps(const RowSpace &rs, int j0, int T, int lane, int entry) {
  const int jb = j0 + lane * KPS;
  const int n_live = min(max(T - jb, 0), KPS);
  int64_t row;
  if (LAYOUT == 0) {
    row = rs.first + jb;
  } else {
    const int64_t blk = rs.blk0 + min(max(entry, 0), rs.n_blocks - 1);  // never leave the pool
    const int64_t in_blk = jb & ((1 << rs.shift) - 1);
    row = LAYOUT == 2 ? ((blk * rs.H + rs.h) << rs.shift) + in_blk : ((blk << rs.shift) + in_blk) * rs.H + rs.h;
  }
  const uint64_t a = reinterpret_cast<uint64_t>(rs.K + row * rs.row_bytes);
  BatchSteps b;
  b.lo = static_cast<uint32_t>(a);
  b.hi = static_cast<uint32_t>(a >> 32);
  b.range = n_live > 0 ? static_cast<int32_t>((n_live - 1) * slot_stride<LAYOUT>(rs) + rs.row_bytes) : 0;
  return b;
}

// Buffer resource of step t (a compile-time lane index into the batch's BatchSteps).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t step_rsrc(const BatchSteps &b, int t) {
  const uint64_t a = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b.hi), t)))
                      << 32) |
                     static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b.lo), t));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(a), 0, __builtin_amdgcn_readlane(b.range, t),
                                           kRowRsrcWord3);
}

__device__ __forceinline__ uint4 load_row_piece(__amdgpu_buffer_rsrc_t r, int lane_off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, 0, kRowLoadNt);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

}  // namespace kvevict

// The memory system's ceiling for the score stream's access pattern (a measurement aid, not part
// of the method): the same loads as tri_score's bf16 head_dim-128 form -- workgroups of 256
// threads over 128 KB each, every wave two batches of sixteen 16-byte pieces per lane, the next
// batch issued before the current one is combined, non-temporal loads -- with no arithmetic but an
// XOR of each lane's pieces, and optionally tri_score's stores (one 4-byte value per 256 bytes
// read, non-temporal). Timed beside tri_score it separates what the access pattern costs from
// what the kernel's arithmetic adds.
#include "kv_internal.hpp"

namespace kvevict {
namespace {

constexpr int kCeilThreads = 256;
constexpr int kCeilBatch = 16 * 1024;            // bytes per wave batch: 16 steps of 1 KB
constexpr int kCeilWaveBytes = 2 * kCeilBatch;   // two batches per wave
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

template <bool STORES>
__global__ __launch_bounds__(kCeilThreads) void stream_ceiling_kernel(const char *buf, uint32_t *out) {
  const int lane = threadIdx.x & 63;
  const long long wave_g = static_cast<long long>(blockIdx.x) * (kCeilThreads / 64) + (threadIdx.x >> 6);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char *>(buf + wave_g * kCeilWaveBytes), 0, kCeilWaveBytes, 0x00020000);
  v4u32 a[16], b[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) a[t] = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, t * 1024, 2);
#pragma unroll
  for (int t = 0; t < 16; ++t) b[t] = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, kCeilBatch + t * 1024, 2);
  uint32_t x = 0u, y = 0u;
#pragma unroll
  for (int t = 0; t < 16; ++t) x ^= a[t][0] ^ a[t][1] ^ a[t][2] ^ a[t][3];
  const long long row = wave_g * (kCeilWaveBytes / 256);   // the wave's first 256-byte row
  if (STORES) __builtin_nontemporal_store(x, out + row + lane);
#pragma unroll
  for (int t = 0; t < 16; ++t) y ^= b[t][0] ^ b[t][1] ^ b[t][2] ^ b[t][3];
  if (STORES) {
    __builtin_nontemporal_store(y, out + row + 64 + lane);
  } else {
    uint32_t v = x ^ y;   // one value per wave: the XOR over its lanes
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off, 64));
    if (lane == 0) out[wave_g] = v;
  }
}

}  // namespace

hipError_t launch_stream_ceiling(const void *buf, size_t bytes, uint32_t *out, bool stores, hipStream_t st) {
  const size_t wg_bytes = static_cast<size_t>(kCeilThreads / 64) * kCeilWaveBytes;
  const dim3 grid(static_cast<unsigned>(bytes / wg_bytes)), blk(kCeilThreads);
  if (stores)
    hipLaunchKernelGGL(stream_ceiling_kernel<true>, grid, blk, 0, st, static_cast<const char *>(buf), out);
  else
    hipLaunchKernelGGL(stream_ceiling_kernel<false>, grid, blk, 0, st, static_cast<const char *>(buf), out);
  return hipGetLastError();
}

}  // namespace kvevict

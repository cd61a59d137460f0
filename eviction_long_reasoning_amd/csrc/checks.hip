// Device-side precondition checks, launched before a call's own kernels by a build with
// KV_DEVICE_CHECKS (libkvevict_debug.so). They compute nothing of the method: each workgroup looks
// at one (layer, sequence, KV head) and ORs into the workspace status word the KV_DEV_* bits of
// what it finds -- a length outside [0, t_cap], a prompt length outside [0, prompt_cap], positions
// that do not strictly ascend over the head's valid slots. The kernels that follow clamp these
// values either way; the word only tells the caller that its data broke a documented rule.
#include "kvevict.h"
#include "kv_internal.hpp"

namespace kvevict {
namespace {

constexpr int kCheckThreads = 256;

__global__ __launch_bounds__(kCheckThreads) void check_kernel(const CheckParams c) {
  __shared__ uint32_t flags;
  const int head = blockIdx.x;
  const int h = head % c.H;
  const int s = (head / c.H) % c.S;
  const int l = head / (c.H * c.S);
  if (threadIdx.x == 0) flags = 0u;
  __syncthreads();
  const int len = c.seq_len[s];
  uint32_t f = 0u;
  if (threadIdx.x == 0 && l == 0 && h == 0) {   // per-sequence values: checked once
    if (len < 0 || len > c.t_cap) f |= KV_DEV_SEQ_LEN;
    if (c.prompt_len) {
      const int pl = c.prompt_len[s];
      if (pl < 0 || pl > c.prompt_cap) f |= KV_DEV_PROMPT_LEN;
    }
  }
  if (c.pos) {
    const int T = min(max(len, 0), c.t_cap);
    const int32_t *row = c.pos + static_cast<size_t>(head) * c.t_cap;
    for (int j = 1 + static_cast<int>(threadIdx.x); j < T; j += kCheckThreads)
      if (row[j] <= row[j - 1]) f |= KV_DEV_POS_ORDER;
  }
  if (f) atomicOr(&flags, f);
  __syncthreads();
  if (threadIdx.x == 0 && flags) atomicOr(c.status, flags);
}

}  // namespace

hipError_t launch_device_checks(const CheckParams &c, hipStream_t st) {
  const long long heads = static_cast<long long>(c.L) * c.S * c.H;
  if (heads <= 0) return hipSuccess;
  hipLaunchKernelGGL(check_kernel, dim3(static_cast<unsigned>(heads)), dim3(kCheckThreads), 0, st, c);
  return hipGetLastError();
}

}  // namespace kvevict

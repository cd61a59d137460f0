// Test helper: prints rocRAND's Philox4x32-10 output for (seed, subsequence, offset) triples
// read from stdin, one block of four words per line. rocRAND's documented stream places the
// subsequence in counter words 2..3, the offset/4 in words 0..1 and the seed in the key, so
// the first block of a fresh state is Philox(ctr=(off/4, 0, sub_lo, sub_hi), key=seed).
// Used only by the oracle's Philox pin test; neither the oracle nor the HIP path links it.
#include <rocrand/rocrand_kernel.h>
#include <cstdio>

int main() {
  unsigned long long seed, sub, off;
  while (std::scanf("%llu %llu %llu", &seed, &sub, &off) == 3) {
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, sub, off, &st);
    uint4 v = rocrand4(&st);
    std::printf("%u %u %u %u\n", v.x, v.y, v.z, v.w);
  }
  return 0;
}

// Independent Philox4x32-10: rocRAND's engine (header-only, host side) evaluated on
// counter/key lines read from stdin, one output block per line on stdout.
// Input line: c0 c1 c2 c3 k0 k1 (decimal uint32); c1 < 2^30.  Output: r0 r1 r2 r3.
// The engine is seeded with key (k0, k1), moved to subsequence c2 + 2^32 c3 (the two
// high counter words) and then forward by 4 (c0 + 2^32 c1) numbers (the two low
// words), so its counter equals (c0, c1, c2, c3) when the block is drawn.
#include <cstdio>
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_philox4x32_10.h>

int main() {
  unsigned c[4], k[2];
  while (std::scanf("%u %u %u %u %u %u", c, c + 1, c + 2, c + 3, k, k + 1) == 6) {
    const unsigned long long seed = (unsigned long long)k[1] << 32 | k[0];
    const unsigned long long sub = (unsigned long long)c[3] << 32 | c[2];
    const unsigned long long blk = (unsigned long long)c[1] << 32 | c[0];
    if (c[1] >= (1u << 30)) return 2;  // 4 * blk must fit 64 bits
    rocrand_device::philox4x32_10_engine e(seed, sub, 0);
    e.discard(4ull * blk);
    const uint4 r = e.next4();
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}

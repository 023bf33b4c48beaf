// Host reference for the oracle's Philox4x32-10 pin: rocRAND's header-only
// engine.  Reads lines "seed subsequence offset" (decimal) and prints the
// four 32-bit words the engine produces there, in hex.  The engine's 128-bit
// counter is (offset / 4 in words 0-1, subsequence in words 2-3) and its key
// is the seed (low word first).
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

int main() {
  unsigned long long seed, sub, off;
  while (std::scanf("%llu %llu %llu", &seed, &sub, &off) == 3) {
    rocrand_device::philox4x32_10_engine e(seed, sub, off);
    const uint4 v = e.next4();
    std::printf("%08x %08x %08x %08x\n", v.x, v.y, v.z, v.w);
  }
  return 0;
}

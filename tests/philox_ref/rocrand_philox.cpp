// Test-only reference: prints rocRAND's Philox4x32-10 (rocrand/rocrand_philox4x32_10.h,
// a source header of the ROCm install) for counters and keys read from stdin, one
// "c0 c1 c2 c3 k0 k1" line each.  The engine takes the key as a 64-bit seed, counter
// words 2-3 as the subsequence and counter words 0-1 as offset / 4.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdint>
#include <cstdio>

int main() {
  unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    unsigned long long seed = (unsigned long long)k0 | ((unsigned long long)k1 << 32);
    unsigned long long subseq = (unsigned long long)c2 | ((unsigned long long)c3 << 32);
    unsigned long long offset = ((unsigned long long)c0 | ((unsigned long long)c1 << 32)) * 4ull;
    rocrand_device::philox4x32_10_engine eng(seed, subseq, offset);
    unsigned a = eng(), b = eng(), c = eng(), d = eng();
    std::printf("%u %u %u %u\n", a, b, c, d);
  }
  return 0;
}

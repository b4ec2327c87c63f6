// Test-only reference: prints PyTorch's Philox4x32-10 (ATen/core/PhiloxRNGEngine.h,
// a header-only source file shipped with torch) for counters and keys read from
// stdin, one "c0 c1 c2 c3 k0 k1" line each.  The engine takes the key as a 64-bit
// seed, counter words 0-1 as the offset and words 2-3 as the subsequence.
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdint>
#include <cstdio>

int main() {
  unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    uint64_t seed = (uint64_t)k0 | ((uint64_t)k1 << 32);
    uint64_t subseq = (uint64_t)c2 | ((uint64_t)c3 << 32);
    uint64_t offset = (uint64_t)c0 | ((uint64_t)c1 << 32);
    at::Philox4_32 eng(seed, subseq, offset);
    unsigned a = eng(), b = eng(), c = eng(), d = eng();
    std::printf("%u %u %u %u\n", a, b, c, d);
  }
  return 0;
}

// Host check of the launch-time division helper used by the decode kernel: compares
// fast_div(n, make_fastdiv(d)) with n / d for every divisor 1..4096 and a sweep of
// numerators (all n < 65536, powers of two and their neighbours, and a pseudo-random sample
// up to 2^32 - 1), plus divisors up to 2^31.  Prints "ok" or the first mismatch.
#include <cstdio>
#include <cstdint>
#include "internal.h"

static int check(uint32_t n, uint32_t d) {
  const mla::FastDiv f = mla::make_fastdiv(d);
  const uint32_t q = mla::fast_div(n, f);
  if (q != n / d) {
    std::printf("mismatch n=%u d=%u got %u want %u\n", n, d, q, n / d);
    return 1;
  }
  return 0;
}

int main() {
  uint64_t x = 0x9E3779B97F4A7C15ull;
  for (uint32_t d = 1; d <= 4096; ++d) {
    for (uint32_t n = 0; n < 65536; n += (d < 64 ? 1 : 7))
      if (check(n, d)) return 1;
    for (int k = 0; k < 32; ++k)
      for (int e = -1; e <= 1; ++e)
        if (check((uint32_t)((1ull << k) + e), d)) return 1;
    if (check(0xFFFFFFFFu, d)) return 1;
    for (int k = 0; k < 64; ++k) {
      x ^= x << 13; x ^= x >> 7; x ^= x << 17;
      if (check((uint32_t)x, d)) return 1;
    }
  }
  for (int k = 12; k < 32; ++k)
    for (int e = -1; e <= 1; ++e) {
      const uint32_t d = (uint32_t)((1ull << k) + e);
      for (int j = 0; j < 4096; ++j) {
        x ^= x << 13; x ^= x >> 7; x ^= x << 17;
        if (check((uint32_t)x, d) || check((uint32_t)j * d + (uint32_t)(x & 1), d)) return 1;
      }
    }
  std::printf("ok\n");
  return 0;
}

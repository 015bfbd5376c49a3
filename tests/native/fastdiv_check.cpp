// Host check of the invariant-divisor constants used by the kernels: for
// many divisors and dividends, fdiv(x, make_fastdiv(d)) == x / d.
#include <cstdio>
#include <cstdlib>
#include <random>

#include "fastdiv.h"

int main() {
  std::mt19937_64 rng(12345);
  long long checked = 0;
  auto check = [&](uint32_t x, uint32_t d) {
    const bra::FastDiv f = bra::make_fastdiv(d);
    const int q = bra::fdiv((int)x, f);
    ++checked;
    if (q != (int)(x / d)) {
      std::printf("FAIL x=%u d=%u got %d want %u\n", x, d, q, x / d);
      std::exit(1);
    }
  };
  for (uint32_t d = 1; d <= 4096; ++d) {
    for (uint32_t x = 0; x < 3 * d + 5; ++x) check(x, d);
    for (uint32_t k : {1u, 2u, 3u, 1000u, 65535u, 524287u})
      for (int dx = -1; dx <= 1; ++dx) {
        const long long x = (long long)k * d + dx;
        if (x >= 0 && x < (1ll << 31)) check((uint32_t)x, d);
      }
    check(0x7fffffffu, d);
    check(0x7ffffffeu, d);
  }
  for (int i = 0; i < 2000000; ++i) {
    const uint32_t d = 1 + (uint32_t)(rng() % 0x7ffffffe);
    const uint32_t x = (uint32_t)(rng() & 0x7fffffff);
    check(x, d);
    check(x, 1 + d % 100000);
  }
  std::printf("ok %lld\n", checked);
  return 0;
}

// Division of non-negative 31-bit integers by a divisor fixed per launch:
// q = (umulhi(x, m) + x) >> s, with s = ceil(log2 d) and
// m = floor(2^32 * (2^s - d) / d) + 1 (the round-up method for division by
// invariant integers of Granlund and Montgomery, 1994).  Exact for every
// 0 <= x < 2^31 and 1 <= d < 2^31; the add cannot overflow 32 bits there.
// Usable from host (to build the constants) and device code.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define BRA_HD __host__ __device__
#else
#define BRA_HD
#endif

namespace bra {

struct FastDiv {
  uint32_t d;   // divisor
  uint32_t m;   // magic multiplier
  uint32_t s;   // shift
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.s = s;
  f.m = (uint32_t)((((1ull << 32) * ((1ull << s) - d)) / d) + 1);
  return f;
}

BRA_HD inline uint32_t umulhi32(uint32_t a, uint32_t b) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __umulhi(a, b);
#else
  return (uint32_t)(((uint64_t)a * b) >> 32);
#endif
}

BRA_HD inline int fdiv(int x, const FastDiv& f) {
  return (int)((umulhi32((uint32_t)x, f.m) + (uint32_t)x) >> f.s);
}

}  // namespace bra

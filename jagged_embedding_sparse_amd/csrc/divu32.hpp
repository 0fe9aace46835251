// Unsigned 32-bit division by a run-time invariant divisor with one high
// multiply, after Granlund and Montgomery, "Division by invariant integers
// using multiplication" (PLDI 1994), section 4: for 1 <= d < 2^32 let
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1 (it fits 32 bits);
// then for every 32-bit n, with t = floor(m n / 2^32),
//   floor(n / d) = (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0).
// Shard ids (id / ceil(rows / W)) are taken this way in the kernels; the host
// builds the constants. Plain C++ so that a host compiler can check it.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define FS_HD __host__ __device__
#else
#define FS_HD
#endif

namespace fs {

struct DivU32 {
  uint32_t m;   // magic multiplier
  uint32_t s1;  // min(l, 1)
  uint32_t s2;  // max(l - 1, 0)
};

// d in [1, 2^32 - 1]
inline DivU32 make_divu32(uint32_t d) {
  uint32_t l = 0;
  while (l < 32 && (1ull << l) < (uint64_t)d) ++l;
  const uint64_t m = (((1ull << 32) * ((1ull << l) - (uint64_t)d)) / (uint64_t)d) + 1;
  DivU32 r;
  r.m = (uint32_t)m;
  r.s1 = l < 1 ? l : 1;
  r.s2 = l > 1 ? l - 1 : 0;
  return r;
}

FS_HD inline uint32_t divu32(uint32_t n, DivU32 q) {
  const uint32_t t = (uint32_t)(((uint64_t)q.m * (uint64_t)n) >> 32);
  return (t + ((n - t) >> q.s1)) >> q.s2;
}

}  // namespace fs

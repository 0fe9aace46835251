// Host check of divu32 against the hardware divide: edge divisors (1, powers
// of two and their neighbours, 2^32 - 1, shard blocks of real table sizes)
// against edge and random numerators. Prints "ok <count>" or the first
// mismatch and exits non-zero.
#include <stdio.h>
#include <stdint.h>

#include "divu32.hpp"

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t next32() {  // splitmix64
  uint64_t z = (state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (uint32_t)((z ^ (z >> 31)) >> 32);
}

static int check(uint32_t d, uint32_t n, uint64_t* count) {
  const uint32_t got = fs::divu32(n, fs::make_divu32(d));
  ++*count;
  if (got != n / d) {
    printf("mismatch d=%u n=%u got=%u want=%u\n", d, n, got, n / d);
    return 1;
  }
  return 0;
}

int main() {
  uint32_t ds[256];
  int nd = 0;
  for (int k = 0; k < 32; ++k) {
    const uint32_t p = 1u << k;
    ds[nd++] = p;
    if (p > 1) ds[nd++] = p - 1;
    ds[nd++] = p + 1;
  }
  ds[nd++] = 0xFFFFFFFFu;
  ds[nd++] = 0xFFFFFFFEu;
  const uint64_t rows[] = {100000, 10000000, 50000000, 200000000, 4294967295ull};
  const int ws[] = {1, 3, 4, 16, 64, 256, 512, 1000, 1024};
  for (uint64_t r : rows)
    for (int w : ws) ds[nd++] = (uint32_t)((r + w - 1) / w);
  while (nd < 256) ds[nd++] = next32() | 1u;
  uint64_t count = 0;
  for (int i = 0; i < nd; ++i) {
    const uint32_t d = ds[i];
    if (d == 0) continue;
    const uint32_t edge[] = {0u, 1u, d - 1, d, d + 1, 2 * d - 1, 2 * d, 0xFFFFFFFFu,
                             0xFFFFFFFEu, 0x80000000u, 0x7FFFFFFFu};
    for (uint32_t n : edge)
      if (check(d, n, &count)) return 1;
    // around multiples of d
    for (int k = 0; k < 64; ++k) {
      const uint64_t mlt = (uint64_t)d * (next32() % (0xFFFFFFFFull / d + 1));
      for (int e = -1; e <= 1; ++e) {
        const int64_t n = (int64_t)mlt + e;
        if (n >= 0 && n <= 0xFFFFFFFFll && check(d, (uint32_t)n, &count)) return 1;
      }
    }
    for (int k = 0; k < 4096; ++k)
      if (check(d, next32(), &count)) return 1;
  }
  // random divisors x random numerators
  for (int k = 0; k < 2000000; ++k) {
    uint32_t d = next32() >> (next32() % 32);
    if (d == 0) d = 1;
    if (check(d, next32(), &count)) return 1;
  }
  printf("ok %llu\n", (unsigned long long)count);
  return 0;
}

// Exhaustive and random checks of the kernels' division by launch constants
// (FastDiv in mgqa_internal.h): (x * m) >> (31 + s) must equal x / d for every
// 0 <= x < 2^31.  Built and run by tests/test_fastdiv.py on the host.
#include <cstdint>
#include <cstdio>
#include <random>

#include "mgqa_internal.h"

int main() {
  std::mt19937 rng(12345);
  long bad = 0, n = 0;
  auto check = [&](uint32_t d, const mgqa::FastDiv& f, uint32_t x) {
    const uint32_t q = (uint32_t)(((uint64_t)x * f.m) >> (31 + f.s));
    ++n;
    if (q != x / d) {
      if (bad < 5) std::printf("mismatch d=%u x=%u got %u want %u\n", d, x, q, x / d);
      ++bad;
    }
  };
  for (uint32_t d = 1; d <= 20000; d += (d < 2048 ? 1 : 61)) {
    const mgqa::FastDiv f = mgqa::make_fastdiv(d);
    for (uint32_t x = 0; x < 20000; ++x) check(d, f, x);
    for (int i = 0; i < 500; ++i) check(d, f, rng() & 0x7FFFFFFFu);
    const uint32_t top = 0x7FFFFFFFu;
    check(d, f, top);
    check(d, f, d * (top / d));
    if (d * (top / d) > 0) check(d, f, d * (top / d) - 1);
  }
  for (uint32_t d : {3u, 7u, 65537u, 0x3FFFFFFFu, 0x40000000u, 0x40000001u, 0x7FFFFFFFu}) {
    const mgqa::FastDiv f = mgqa::make_fastdiv(d);
    for (int i = 0; i < 100000; ++i) check(d, f, rng() & 0x7FFFFFFFu);
  }
  std::printf("checked %ld quotients, %ld wrong\n", n, bad);
  return bad != 0;
}

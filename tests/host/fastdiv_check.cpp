// Host-side check of the library's division by an invariant integer (used on
// the device for p mod P and floor(p / s)): compares against plain integer
// division over divisors 1..5000 and selected large ones, for dense small
// numerators, numerators near multiples of the divisor and the top of the
// non-negative int32 range. Prints "ok <count>" or the first mismatch.
#include <cstdint>
#include <cstdio>

#include "common.hpp"

int main() {
  using namespace prope;
  uint64_t checked = 0;
  auto check = [&](uint32_t n, uint32_t d, const FastDiv& f) {
    const uint32_t q = fastdiv(n, f), r = fastmod(n, f);
    ++checked;
    if (q != n / d || r != n % d) {
      std::printf("mismatch n=%u d=%u got %u,%u want %u,%u\n", n, d, q, r, n / d, n % d);
      return false;
    }
    return true;
  };
  const uint32_t top = 0x7fffffffu;
  for (uint32_t d = 1; d <= 5000; ++d) {
    const FastDiv f = make_fastdiv(d);
    for (uint32_t n = 0; n < 3000; ++n)
      if (!check(n, d, f)) return 1;
    for (uint32_t k = 1; k < 200; ++k) {
      const uint64_t m = uint64_t(k) * 104729u * d;
      for (int e = -1; e <= 1; ++e) {
        const int64_t n = int64_t(m % (uint64_t(top) + 1)) + e;
        if (n >= 0 && n <= top && !check(uint32_t(n), d, f)) return 1;
      }
    }
    for (uint32_t n = top - 2000; n != 0 && n <= top; ++n)
      if (!check(n, d, f)) return 1;
  }
  const uint32_t big[] = {32768u, 65535u, 65536u, 1000003u, 1u << 20, (1u << 30) - 1, 1u << 30,
                          (1u << 30) + 1, top - 1, top, 1u << 31};
  for (uint32_t d : big) {
    const FastDiv f = make_fastdiv(d);
    uint64_t x = 88172645463325252ull;
    for (int i = 0; i < 200000; ++i) {
      x ^= x << 13; x ^= x >> 7; x ^= x << 17;
      if (!check(uint32_t(x & top), d, f)) return 1;
    }
    for (uint32_t n = top - 1000; n != 0 && n <= top; ++n)
      if (!check(n, d, f)) return 1;
  }
  std::printf("ok %llu\n", static_cast<unsigned long long>(checked));
  return 0;
}

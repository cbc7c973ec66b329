// Host-side check of the library's division by an invariant integer (used on
// the device for p mod P and floor(p / s)): compares against plain integer
// division over divisors 1..5000 and selected large ones, for dense small
// numerators, numerators near multiples of the divisor and the top of the
// non-negative int32 range. The signed forms (floor semantics for negative
// ids) are compared with 64-bit floor division over the whole int32 range's
// edges, and the 64-bit multiply-divide (interpolated frequencies) with a
// 128-bit product; the rotation phase from the signed split of the frequency
// word against 64-bit wrap-around arithmetic. Prints "ok <count>" or the first
// mismatch.
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
  // signed floor division and modulo
  auto check_s = [&](int32_t n, uint32_t d, const FastDiv& f) {
    const int64_t q = int64_t(n) >= 0 ? int64_t(n) / d : -((-int64_t(n) + d - 1) / int64_t(d));
    const int64_t r = int64_t(n) - q * int64_t(d);
    ++checked;
    if (floordiv_s(n, f) != q || floormod_s(n, f) != r || r < 0 || r >= int64_t(d)) {
      std::printf("signed mismatch n=%d d=%u got %d,%d want %lld,%lld\n", n, d, floordiv_s(n, f),
                  floormod_s(n, f), (long long)q, (long long)r);
      return false;
    }
    return true;
  };
  for (uint32_t d = 1; d <= 3000; ++d) {
    const FastDiv f = make_fastdiv(d);
    for (int32_t n = -4000; n <= 4000; ++n)
      if (!check_s(n, d, f)) return 1;
    for (int32_t e = 0; e < 300; ++e)
      if (!check_s(INT32_MIN + e, d, f) || !check_s(INT32_MAX - e, d, f)) return 1;
  }
  for (uint32_t d : big) {
    if (d > 0x7fffffffu) continue;
    const FastDiv f = make_fastdiv(d);
    uint64_t x = 0x9e3779b97f4a7c15ull;
    for (int i = 0; i < 200000; ++i) {
      x ^= x << 13; x ^= x >> 7; x ^= x << 17;
      if (!check_s(static_cast<int32_t>(static_cast<uint32_t>(x)), d, f)) return 1;
    }
    for (int32_t e = 0; e < 1000; ++e)
      if (!check_s(INT32_MIN + e, d, f)) return 1;
  }
  // 64-bit multiply-divide: floor(F * num / den) for num <= den < 2^31
  {
    uint64_t x = 0x243f6a8885a308d3ull;
    auto next = [&]() { x ^= x << 13; x ^= x >> 7; x ^= x << 17; return x; };
    for (int i = 0; i < 2000000; ++i) {
      const uint64_t F = next();
      uint32_t den = static_cast<uint32_t>(next() & 0x7fffffffu);
      if (den == 0) den = 1;
      if (i % 3 == 0) den = 1 + static_cast<uint32_t>(next() % 300000);  // sequence lengths
      const uint32_t num = 1 + static_cast<uint32_t>(next() % den);
      const unsigned __int128 want = (static_cast<unsigned __int128>(F) * num) / den;
      ++checked;
      if (muldiv_u64(F, num, den) != static_cast<uint64_t>(want)) {
        std::printf("muldiv mismatch F=%llu num=%u den=%u\n", (unsigned long long)F, num, den);
        return 1;
      }
    }
  }
  // the rotation phase from the signed split of F: top 32 bits of (r * F) mod 2^64
  // for sign-extended r, against plain 64-bit wrap-around arithmetic
  {
    uint64_t x = 0x9e3779b97f4a7c15ull;
    auto next = [&]() { x ^= x << 13; x ^= x >> 7; x ^= x << 17; return x; };
    const int32_t edge_r[] = {INT32_MIN, INT32_MIN + 1, -65537, -1, 0, 1, 2, 65536, INT32_MAX - 1, INT32_MAX};
    const uint64_t edge_f[] = {0ull, 1ull, 0x7fffffffull, 0x80000000ull, 0xffffffffull, 0x100000000ull,
                               0x80000000ffffffffull, 0xffffffff80000000ull, ~0ull};
    auto check_p = [&](int32_t r, uint64_t F) {
      const uint32_t want = static_cast<uint32_t>((static_cast<uint64_t>(static_cast<int64_t>(r)) * F) >> 32);
      const PhaseSplit sp = phase_split(static_cast<uint32_t>(F), static_cast<uint32_t>(F >> 32));
      ++checked;
      if (phase_top_split(r, sp.fls, sp.fhs) != want) {
        std::printf("phase mismatch r=%d F=%llu\n", r, (unsigned long long)F);
        return false;
      }
      return true;
    };
    for (int32_t r : edge_r)
      for (uint64_t F : edge_f)
        if (!check_p(r, F)) return 1;
    for (int i = 0; i < 2000000; ++i) {
      const uint64_t a = next(), F = next();
      if (!check_p(static_cast<int32_t>(a), F)) return 1;
    }
  }
  std::printf("ok %llu\n", static_cast<unsigned long long>(checked));
  return 0;
}

// Host check of the library's run-time-invariant integer division (rope_plan.h): compares
// fastdiv_host(make_fastdiv(d), n) with n / d over every divisor up to 70000 with a spread of
// dividends, powers of two and their neighbours, and random 32-bit pairs, plus every n for a
// few divisors.  Prints "ok <count>" or the first counterexample; exit status 1 on failure.
// An optional argument k > 1 keeps every k-th divisor and a k times sparser sweep of n (for
// runs under the sanitizers, which check the arithmetic for undefined behaviour).
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "rope_plan.h"

using ropeamd::fastdiv_host;
using ropeamd::make_fastdiv;

static uint64_t s = 0x9E3779B97F4A7C15ull;
static uint32_t rnd() {
  s ^= s << 13; s ^= s >> 7; s ^= s << 17;
  return uint32_t(s >> 11);
}

int main(int argc, char **argv) {
  const uint32_t k_stride = argc > 1 ? uint32_t(std::atoi(argv[1])) : 1u;
  const uint32_t stride = k_stride > 0 ? k_stride : 1u;
  uint64_t checks = 0;
  auto check = [&](uint32_t d, uint32_t n) {
    const ropeamd::FastDiv f = make_fastdiv(d);
    const uint32_t q = fastdiv_host(f, n);
    ++checks;
    if (q != n / d) {
      std::printf("FAIL d=%u n=%u got %u want %u\n", d, n, q, n / d);
      return false;
    }
    return true;
  };
  std::vector<uint32_t> ns = {0u, 1u, 2u, 3u, 0x7fffffffu, 0x80000000u, 0xfffffffeu, 0xffffffffu};
  for (int b = 0; b < 32; ++b) {
    ns.push_back(1u << b);
    ns.push_back((1u << b) - 1);
    ns.push_back((1u << b) + 1);
  }
  for (uint32_t d = 1; d <= 70000; d += stride) {
    for (uint32_t n : ns) if (!check(d, n)) return 1;
    for (int k = 0; k < 64; ++k) {
      const uint32_t n = rnd();
      if (!check(d, n)) return 1;
      const uint32_t m = (n / d) * d;  // around multiples of d
      if (!check(d, m) || (m > 0 && !check(d, m - 1)) || (m < 0xffffffffu && !check(d, m + 1)))
        return 1;
    }
  }
  std::vector<uint32_t> ds = {0x7fffffffu, 0x80000000u, 0x80000001u, 0xfffffffeu, 0xffffffffu};
  for (int b = 0; b < 32; ++b) {
    ds.push_back(1u << b);
    ds.push_back((1u << b) + 1);
    if (b > 1) ds.push_back((1u << b) - 1);
  }
  for (uint32_t k = 0; k < 4000 / stride; ++k) ds.push_back(rnd() | 1u);
  for (uint32_t d : ds) {
    for (uint32_t n : ns) if (!check(d, n)) return 1;
    for (int k = 0; k < 2000; ++k) if (!check(d, rnd())) return 1;
  }
  for (uint32_t d : {3u, 7u, 40u, 320u, 1000003u}) {
    for (uint64_t n = 0; n <= 0xffffffffull; n += uint64_t(d == 3u ? 1 : 4099) * stride) {
      if (!check(d, uint32_t(n))) return 1;
    }
  }
  std::printf("ok %llu\n", (unsigned long long)checks);
  return 0;
}

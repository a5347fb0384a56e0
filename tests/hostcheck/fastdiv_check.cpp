// Host-side check of the launch-constant divisors (FastDiv in csrc/common.h):
// the multiply-and-shift quotient against the integer division, for every
// divisor up to 4096 over the dividends 0..70,000, the multiples of the
// divisor and their neighbours near 2^31, and random (divisor, dividend)
// pairs over the whole range.  Exit status 0 when every quotient matches.
#include <cstdint>
#include <cstdio>
#include <random>

#include "common.h"

int main() {
  using ddt::FastDiv;
  long bad = 0, total = 0;
  auto check = [&](uint32_t d, int n) {
    const FastDiv f = ddt::make_fastdiv(d);
    int rem = 0;
    const int q = ddt::fdivmod(n, f, rem);
    ++total;
    if (q != (int)((uint32_t)n / d) || rem != (int)((uint32_t)n % d)) {
      if (bad < 5) std::printf("mismatch d=%u n=%d q=%d\n", d, n, q);
      ++bad;
    }
  };
  std::mt19937_64 g(20240601);
  for (uint32_t d = 1; d <= 4096; ++d) {
    for (int n = 0; n < 70000; ++n) check(d, n);
    for (int i = 0; i < 256; ++i) {
      const long top = 0x7FFFFFFFL - i;
      check(d, (int)top);
      const long m = (0x7FFFFFFFL / d - i) * (long)d;
      if (m >= 0) check(d, (int)m);
      if (m > 0) check(d, (int)(m - 1));
    }
  }
  for (int i = 0; i < 4000000; ++i) {
    uint32_t d = (uint32_t)(g() % 0x7FFFFFFFu) + 1u;
    d >>= (unsigned)(g() % 31);
    check(d == 0 ? 1u : d, (int)(g() & 0x7FFFFFFFu));
  }
  std::printf("checked %ld quotients, %ld mismatches\n", total, bad);
  return bad == 0 ? 0 : 1;
}

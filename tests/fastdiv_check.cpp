// Host check of the multiply-shift division the small kernels use instead
// of integer divides (FastDiv / fdiv): exact floor(n / d) wherever the
// kernels apply it.  Built and run by test_fastdiv.py; prints the number of
// cases checked, or the first failing (n, d) and exits nonzero.
#include <cstdint>
#include <cstdio>
#include <random>

#include "device.h"

static long long checked = 0;

static bool check(int n, int d) {
  const miep::FastDiv f = miep::make_fastdiv(d);
  ++checked;
  if (miep::fdiv(n, f) != n / d) {
    std::printf("FAIL n=%d d=%d fdiv=%d floor=%d\n", n, d, miep::fdiv(n, f), n / d);
    return false;
  }
  return true;
}

int main() {
  // exhaustive: every divisor up to 256, every numerator below 2^16
  for (int d = 1; d <= 256; ++d)
    for (int n = 0; n < (1 << 16); ++n)
      if (!check(n, d)) return 1;
  // expert / experts-per-rank: both below 8192, every divisor, the numerators
  // around each multiple (where a rounding error would show first)
  for (int d = 1; d <= 8192; ++d)
    for (int q = 0; q * d < 8192 + d; ++q)
      for (int e : {q * d - 1, q * d, q * d + 1, q * d + d - 1})
        if (e >= 0 && e < 8192 && !check(e, d)) return 1;
  // token / tokens-per-channel for T <= 2^20 tokens, tc = ceil(T / C) <= T:
  // numerators near the multiples of tc, at the ends of the range
  std::mt19937_64 rng(7);
  for (int it = 0; it < 200000; ++it) {
    const int T = 1 + static_cast<int>(rng() % (1u << 20));
    const int C = 1 + static_cast<int>(rng() % 1024);
    const int tc = (T + C - 1) / C;
    const int k = static_cast<int>(rng() % (T / tc + 1));
    for (int n : {k * tc - 1, k * tc, k * tc + 1, k * tc + tc - 1, T - 1})
      if (n >= 0 && n < T && !check(n, tc)) return 1;
  }
  for (int tc : {1, 2, 3, 1023, 1024, 1025, (1 << 20) - 1, 1 << 20})
    for (int n : {0, tc - 1, tc, (1 << 20) - 1})
      if (n >= 0 && n < (1 << 20) && !check(n, tc)) return 1;
  std::printf("ok %lld\n", checked);
  return 0;
}

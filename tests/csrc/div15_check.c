/* The mlx4g32 encoder computes range / 15 as q = fl(range * c), c = fl(1/15), then
 * fl(q + fma(-q, 15, range) * c) with two fused multiply-adds. This program compares that
 * with the correctly rounded fp32 quotient for every fp32 value in [2^lo, 2^hi) (the
 * exponents given on the command line) and for zero, and prints the mismatch count. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int main(int argc, char **argv) {
  const int lo = argc > 1 ? atoi(argv[1]) : -26, hi = argc > 2 ? atoi(argv[2]) : 18;
  const float c = 1.0f / 15.0f;
  float a = ldexpf(1.0f, lo), b = ldexpf(1.0f, hi);
  uint32_t ua, ub;
  memcpy(&ua, &a, 4);
  memcpy(&ub, &b, 4);
  unsigned long long bad = 0, n = 0;
  for (uint64_t u = ua; u < ub; ++u, ++n) {
    float x;
    const uint32_t v = (uint32_t)u;
    memcpy(&x, &v, 4);
    const float q = x * c;
    const float s = fmaf(fmaf(-q, 15.0f, x), c, q);
    if (s != x / 15.0f) ++bad;
  }
  {
    const float x = 0.0f, q = x * c;
    if (fmaf(fmaf(-q, 15.0f, x), c, q) != x / 15.0f) ++bad;
    ++n;
  }
  printf("%llu %llu\n", n, bad);
  return 0;
}

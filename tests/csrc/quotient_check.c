/* Exhaustive check of the reciprocal-based quotient used by the bf16
 * quantization kernels.
 *
 * For every positive finite bf16 absmax a and every bf16 x with 0 <= x <= a
 * (the sign is symmetric), with s = fl32(a / 127) and, when s >= 2^-96,
 * r = fl32(1 / s), q = fl32(x * r), q' = fma(fma(-q, s, x), r, q):
 *   rne(q') == clamp(rne(fl32(x / s)), -127, 127)
 * with no clamp of q' (the int8 kernels take none on this path: s is a
 * normal number within 2^-24 of a / 127, so q' <= a / s stays below 127.5),
 * and adding 1.5 * 2^23 to q' rounds it to that integer, half to even, with
 * its two's-complement byte in the low byte of the sum's bit pattern.
 * With the argument "448" (the FP8 kernels: s = fl32(a / 448), codes OCP
 * e4m3) it checks instead that q' and fl32(x / s), each clamped to 448 and
 * rounded to the e4m3 grid (round half to even, subnormal step 2^-9), give
 * the same value.  (The quotients themselves differ in the last bit on about
 * 0.2% of the pairs; the e4m3 codes never do.)
 * Prints "pairs N mismatches M" and exits 0 iff M == 0.  Compile with
 * -O2 -ffp-contract=off -fopenmp (fmaf must be the fused operation). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf16(uint32_t b) {
  uint32_t u = b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint32_t bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

/* nonnegative v clamped to 448 and rounded to the e4m3 grid, half to even */
static double e4m3_grid(float v) {
  double a = v > 448.0f ? 448.0 : (double)v;
  if (a == 0.0) return 0.0;
  int E;
  frexp(a, &E);
  int e = E - 1;
  if (e < -6) e = -6;
  const double step = ldexp(1.0, e - 3);
  return nearbyint(a / step) * step;
}

int main(int argc, char** argv) {
  long long pairs = 0, bad = 0;
  const float min_scale = 0x1p-96f;
  const int fp8 = argc > 1 && strcmp(argv[1], "448") == 0;
  const float divisor = fp8 ? 448.0f : 127.0f;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, bad)
  for (int a = 1; a < 0x7F80; ++a) {
    const float amax = bf16((uint32_t)a);
    const float s = amax / divisor;
    if (!(s >= min_scale)) continue;
    const float r = 1.0f / s;
    for (int xb = 0; xb <= a; ++xb) {
      const float x = bf16((uint32_t)xb);
      if (fp8) {
        /* the kernels give the corrected quotient the sign of x (which also
         * keeps x = -0 at -0, as the division does); for x >= 0 that is the
         * identity, and the negative half mirrors this one */
        const float q = x * r;
        const float t = copysignf(fmaf(fmaf(-q, s, x), r, q), x);
        ++pairs;
        if (e4m3_grid(t) != e4m3_grid(x / s)) ++bad;
        continue;
      }
      float want = rintf(x / s);
      want = fminf(fmaxf(want, -127.0f), 127.0f);
      const float q = x * r;
      const float t = fmaf(fmaf(-q, s, x), r, q);
      const uint32_t w = bits(t + 12582912.0f);
      const int code = (int)(int8_t)(w & 0xFFu);
      ++pairs;
      if ((float)code != want || rintf(t) != want) ++bad;
    }
  }
  printf("pairs %lld mismatches %lld\n", pairs, bad);
  return bad == 0 ? 0 : 1;
}

/* Exhaustive CPU check of the division scheme used by the quantize kernel.
 *
 * The kernel needs rne(fl32(x / s)) for every element of a row, where
 * s = fl32(amax / 127).  Instead of a full IEEE division per element it
 * computes r = fl32(1 / s) once per row and then, per element,
 *     q0 = fl32(x * r);  e = fma(-q0, s, x);  q = fma(e, r, q0)
 * (one reciprocal-based correction step, Markstein's scheme as presented in
 * Muller et al., "Handbook of Floating-Point Arithmetic").  Rows whose scale
 * is below 2^-100 are first multiplied, x and s alike, by 2^100 (exact), so
 * that 1/s cannot overflow.  This program runs that scheme for every finite
 * bf16 amax > 0 and every finite bf16 x with |x| <= amax, and counts the
 * pairs where its integer code differs from the one the correctly rounded
 * quotient gives.  Codes are odd in x and so is every step, so x >= 0 is
 * enough.  Exit status 0 iff there is no mismatch.
 *
 * With the argument "fp8" the divisor is 448 (the largest e4m3 value, the
 * scale of the fp8 variant, s = fl32(amax / 448)) and the codes compared are
 * the e4m3 values the two quotients round to (nearest, ties to even, from the
 * format's definition: 3 mantissa bits, minimum normal 2^-6, subnormal
 * spacing 2^-9, largest value 448).  The scheme's quotient can be one fp32
 * ulp off only for subnormal x, where it is far below half the smallest e4m3
 * subnormal and both round to zero.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf16(uint32_t bits) { uint32_t u = bits << 16; float f; memcpy(&f, &u, 4); return f; }

static float code_ref(float x, float s) {
  float q = rintf(x / s);
  return fminf(fmaxf(q, -127.0f), 127.0f);
}

static float code_fast(float x, float s, float r) {
  float q0 = x * r;
  float e = fmaf(-q0, s, x);
  float q = fmaf(e, r, q0);
  return fminf(fmaxf(rintf(q), -127.0f), 127.0f);
}

/* nearest e4m3 value of a >= 0 (ties to even mantissa), saturating at 448 */
static float e4m3(float a) {
  if (a >= 464.0f) return 448.0f;
  if (a < 0x1p-6f) return rintf(a * 0x1p9f) * 0x1p-9f;
  int e;
  frexpf(a, &e);                 /* a = f * 2^e, 0.5 <= f < 1 */
  const float spacing = ldexpf(1.0f, e - 4);
  return rintf(a / spacing) * spacing;
}

static float quot_fast(float x, float s, float r) {
  float q0 = x * r;
  float e = fmaf(-q0, s, x);
  return fmaf(e, r, q0);
}

int main(int argc, char** argv) {
  const int fp8 = argc > 1 && strcmp(argv[1], "fp8") == 0;
  const float qmax = fp8 ? 448.0f : 127.0f;
  long long pairs = 0, bad = 0, scaled_rows = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, bad, scaled_rows)
  for (uint32_t ab = 1; ab < 0x7F80; ab++) {
    float amax = bf16(ab);
    float s = amax / qmax;
    float xs = 1.0f, ss = s;
    if (s < 0x1p-100f) { xs = 0x1p100f; ss = s * 0x1p100f; scaled_rows++; }
    float r = 1.0f / ss;
    for (uint32_t xb = 0; xb <= ab; xb++) {
      float x = bf16(xb);
      float a = fp8 ? e4m3(x / s) : code_ref(x, s);
      float b = fp8 ? e4m3(quot_fast(x * xs, ss, r)) : code_fast(x * xs, ss, r);
      pairs++;
      if (a != b) {
        if (bad < 10) printf("mismatch amax=%a x=%a ref=%g fast=%g\n", amax, x, a, b);
        bad++;
      }
    }
  }
  printf("pairs=%lld scaled_rows=%lld mismatches=%lld\n", pairs, scaled_rows, bad);
  return bad != 0;
}

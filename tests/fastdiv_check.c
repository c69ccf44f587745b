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

int main(void) {
  long long pairs = 0, bad = 0, scaled_rows = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, bad, scaled_rows)
  for (uint32_t ab = 1; ab < 0x7F80; ab++) {
    float amax = bf16(ab);
    float s = amax / 127.0f;
    float xs = 1.0f, ss = s;
    if (s < 0x1p-100f) { xs = 0x1p100f; ss = s * 0x1p100f; scaled_rows++; }
    float r = 1.0f / ss;
    for (uint32_t xb = 0; xb <= ab; xb++) {
      float x = bf16(xb);
      float a = code_ref(x, s);
      float b = code_fast(x * xs, ss, r);
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

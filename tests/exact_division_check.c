/* Exhaustive check of the division identity used by the fast activation
 * encoder: with y = RN(1/d), q = RN(a * y), r = RN(a - d * q) (a fused
 * multiply-add, exact here) and q' = RN(q + r * y), q' equals RN(a / d)
 * (P. Markstein, IBM J. Res. Dev. 34(1), 1990).
 *
 *  1. a = every positive finite bf16 value (a block maximum), d = 6;
 *  2. a = every binary32 significand in [1, 2), d = every E4M3 significand
 *     1 + m/8.  Scaling a and d by powers of two scales y, q, r and q'
 *     exactly while everything stays in the normal range, so this covers the
 *     per-element factor g_enc / s_dec for g_enc in [2^-60, 2^60].
 * Prints the mismatch counts; exit status 0 only if both are zero. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bits_to_float(uint32_t b) {
  float f;
  memcpy(&f, &b, 4);
  return f;
}

static int same(float a, float b) { return memcmp(&a, &b, 4) == 0; }

static float div_markstein(float a, float d, float y) {
  const float q = a * y;
  const float r = fmaf(-d, q, a);
  return fmaf(r, y, q);
}

int main(void) {
  volatile float six = 6.0f;
  const float y6 = 1.0f / six;
  long bad1 = 0;
  for (uint32_t h = 0; h < 0x7F80u; ++h) {
    const float b = bits_to_float(h << 16);
    if (!same(div_markstein(b, six, y6), b / six)) ++bad1;
  }
  long bad2 = 0;
  for (int m = 0; m < 8; ++m) {
    volatile float d = 1.0f + (float)m / 8.0f;
    const float y = 1.0f / d;
    for (uint32_t s = 0; s < (1u << 23); ++s) {
      const float a = bits_to_float(0x3F800000u | s);
      if (!same(div_markstein(a, d, y), a / d)) ++bad2;
    }
  }
  printf("bf16/6 mismatches %ld\nsignificand/E4M3 mismatches %ld\n", bad1, bad2);
  return (bad1 == 0 && bad2 == 0) ? 0 : 1;
}

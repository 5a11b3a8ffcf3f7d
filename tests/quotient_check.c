/* The activation quantisation computes v / s for the 32 values of a 1x128
 * group from one reciprocal: y = RN(1/s), q0 = RN(v y), q = RN(q0 + y r) with
 * r = v - q0 s exact by fma, the sign of v kept.  This program checks it
 * against the IEEE quotient for every bf16 group maximum amax with
 * s = RN(amax / 448) >= 2^-64 and every bf16 value v with |v| <= amax:
 * the fp32 results must agree wherever |v / s| >= 2^-10, and the e4m3
 * codes (round to nearest even after clamping to +-448, the sign of zero
 * kept) everywhere.  Prints the counts; exit status 0 when both hold. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float e4m3_value[127];  /* the non-negative finite codes 0x00..0x7E */

static int e4m3_code(float x) { /* nearest code, ties to the even code */
  const float a = fabsf(x);
  int best = 0;
  float bd = INFINITY;
  for (int c = 0; c < 127; ++c) {
    const float dd = fabsf(e4m3_value[c] - a);
    if (dd < bd || (dd == bd && (c & 1) == 0)) { bd = dd; best = c; }
  }
  return (signbit(x) ? 0x80 : 0) | best;
}

static float clamp448(float x) { return fminf(fmaxf(x, -448.0f), 448.0f); }

int main(void) {
  for (int c = 0; c < 127; ++c) {
    const int e = c >> 3, m = c & 7;
    e4m3_value[c] = e == 0 ? ldexpf((float)m / 8.0f, -6) : ldexpf(1.0f + (float)m / 8.0f, e - 7);
  }
  long pairs = 0, fp32_diff = 0, fp32_diff_relevant = 0, code_diff = 0;
  for (uint32_t ab = 1; ab < 0x7f80; ++ab) {          /* positive finite bf16 maxima */
    const float amax = f_of(ab << 16);
    const float s = amax / 448.0f;
    if (!(s >= 0x1p-64f)) continue;
    const float y = 1.0f / s;
    for (uint32_t vb = 0; vb < 0x10000; ++vb) {
      const float v = f_of(vb << 16);
      if (!(fabsf(v) <= amax)) continue;
      const float q = v / s;
      const float q0 = v * y;
      const float q1 = copysignf(fmaf(fmaf(-q0, s, v), y, q0), v);
      ++pairs;
      if (u_of(q1) == u_of(q)) continue;
      ++fp32_diff;
      if (fabsf(q) >= 0x1p-10f) ++fp32_diff_relevant;
      if (e4m3_code(clamp448(q)) != e4m3_code(clamp448(q1))) ++code_diff;
    }
  }
  printf("pairs %ld fp32_differ %ld fp32_differ_at_or_above_2^-10 %ld code_differ %ld\n", pairs,
         fp32_diff, fp32_diff_relevant, code_diff);
  return (fp32_diff_relevant == 0 && code_diff == 0) ? 0 : 1;
}

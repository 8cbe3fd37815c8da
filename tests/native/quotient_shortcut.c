/* Exhaustive host check of the quantizers' quotient shortcut.
 *
 * The kernels compute x / s as q0 = x * r, e = fma(-q0, s, x), q = copysign(fma(e, r, q0), x)
 * with r = 1/s (an IEEE division once per row). For every bf16 x with |x| <= amax (both
 * signs, including -0) and every bf16 amax (floored at 1e-8), with s = amax / qmax for
 * qmax in {448, 127}, this program compares q with the IEEE quotient x / s and counts the
 * pairs where they differ while |x / s| >= 2^-11 (a difference there could change an FP8
 * or INT8 code) or where they differ in sign. Both counts must be zero.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(int argc, char** argv) {
  const float qmax = argc > 1 ? (float)atof(argv[1]) : 448.0f;
  unsigned long long pairs = 0, differ = 0, harmful = 0, signflip = 0;
#pragma omp parallel for reduction(+ : pairs, differ, harmful, signflip) schedule(dynamic, 64)
  for (int a = 0; a < 0x7F81; ++a) {          /* every finite bf16 amax, and +inf */
    const float amax = u2f((uint32_t)a << 16);
    const float am = amax < 1e-8f ? 1e-8f : amax;
    volatile float qm = qmax;
    const float s = am / qm;
    const float r = 1.0f / s;
    if (!isfinite(s)) continue;                 /* the kernels divide directly then */
    for (int b = 0; b <= 2 * (a < 0x7F80 ? a : 0x7F7F) + 1; ++b) {
      const float x = u2f(((uint32_t)(b >> 1) << 16) | ((uint32_t)(b & 1) << 31));
      const float ref = x / s;
      const float q0 = x * r;
      const float e = fmaf(-q0, s, x);
      const float q = copysignf(fmaf(e, r, q0), x);
      ++pairs;
      if (f2u(q) != f2u(ref)) {
        ++differ;
        if (fabsf(ref) >= 0x1p-11f || fabsf(q) >= 0x1p-11f) ++harmful;
        if (signbit(q) != signbit(ref)) ++signflip;
      }
    }
  }
  printf("qmax=%g pairs=%llu differ=%llu harmful=%llu signflip=%llu\n", qmax, pairs, differ,
         harmful, signflip);
  return (harmful == 0 && signflip == 0 && pairs > 1000000000ull) ? 0 : 1;
}

/* Exhaustive host check of the FMA-corrected quotient for an arbitrary fp32 scale.
 *
 * q0 = x * r, e = fma(-q0, s, x), q = fma(e, r, q0) with r = 1/s (IEEE). Scaling x or s by a
 * power of two scales every intermediate by the same power as long as all stay normal, so
 * the comparison with the IEEE quotient x / s only depends on the significands. This
 * program runs every bf16 significand of x (8 bits) against every fp32 significand of s
 * (24 bits), both in [1, 2), and counts the pairs where q and x / s differ in any bit. The
 * count must be zero: then the shortcut equals IEEE division wherever the quotient is a
 * normal number, and outside that range every E4M3FN / INT8 code is a zero of the sign of
 * x (tiny quotients, which the kernels give that sign with copysign) or a saturated code
 * (huge ones) either way.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(void) {
  unsigned long long pairs = 0, differ = 0;
#pragma omp parallel for reduction(+ : pairs, differ) schedule(dynamic, 4096)
  for (uint32_t ms = 0; ms < (1u << 23); ++ms) {
    const float s = u2f(0x3F800000u | ms);              /* [1, 2) */
    const float r = 1.0f / s;
    for (uint32_t mx = 0; mx < 128; ++mx) {
      const float x = u2f(0x3F800000u | (mx << 16));    /* bf16 significands in [1, 2) */
      const float q0 = x * r;
      const float e = fmaf(-q0, s, x);
      const float q = fmaf(e, r, q0);
      ++pairs;
      if (f2u(q) != f2u(x / s)) ++differ;
    }
  }
  printf("pairs=%llu differ=%llu\n", pairs, differ);
  return (differ == 0 && pairs == (128ull << 23)) ? 0 : 1;
}

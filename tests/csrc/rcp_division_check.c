/* Exhaustive check behind the MLA kernel's query quantisation: for every
 * fp32 significand of a divisor s in [1, 2) and every bf16 significand of a
 * numerator x in [1, 2), the estimate q0 = RN(x * RN(1/s)) corrected once by
 * its exact remainder, q1 = RN(q0 + RN(x - s q0) * RN(1/s)) (both steps fused
 * multiply-adds), equals the correctly rounded quotient RN(x / s).  Away from
 * overflow and underflow every rounding step scales with the exponents of x
 * and s, so the significands decide.  Prints the counts and exits non-zero
 * on any difference. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(void) {
  long wrong_q0 = 0, wrong_q1 = 0;
#pragma omp parallel for reduction(+ : wrong_q0, wrong_q1) schedule(static)
  for (long m = 0; m < (1l << 23); ++m) {
    const float s = f_of((127u << 23) | (uint32_t)m);
    const float r = 1.0f / s;
    for (uint32_t f = 0; f < 128; ++f) {
      const float x = f_of((127u << 23) | (f << 16));
      const float exact = x / s;
      const float q0 = x * r;
      const float q1 = fmaf(fmaf(-s, q0, x), r, q0);
      wrong_q0 += u_of(q0) != u_of(exact);
      wrong_q1 += u_of(q1) != u_of(exact);
    }
  }
  printf("pairs %ld estimate_wrong %ld corrected_wrong %ld\n", (1l << 23) * 128, wrong_q0, wrong_q1);
  return wrong_q1 != 0;
}

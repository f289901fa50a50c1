/* Exhaustive check of the quantizers' quotient (div_by_scale in the library's
 * common.hpp): for every bf16 amax a > 0 (finite, subnormals included), every
 * bf16 x with |x| <= a, and FMAX in {448, 57344}:
 *   s  = f32(max(a, 1e-12) / FMAX),  r = f32(1 / s)
 *   q0 = f32(x * r),  e' = fma(q0, s, -x),  q = fma(-e', r, q0)
 * is compared with the IEEE quotient f32(x / s).  Prints, per FMAX, the number
 * of pairs, how many differ at all, and how many differ where either value is
 * at least half the format's smallest subnormal (2^-10 for e4m3, 2^-17 for
 * e5m2): only those could change an 8-bit code.  It also counts the pairs where
 * q differs in any bit from the earlier form copysign(fma(e, r, q0), x) with
 * e = fma(-q0, s, x) (the residual's sign makes the copysign unnecessary: e' is
 * -e exactly, and -0 and +0 inputs keep their sign through the final fma). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf16(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

int main(void) {
  const float fmaxes[2] = {448.0f, 57344.0f};
  const float half_min_code[2] = {1.0f / 1024.0f, 1.0f / 131072.0f};
  for (int t = 0; t < 2; ++t) {
    const float FM = fmaxes[t], thr = half_min_code[t];
    long long pairs = 0, differ = 0, differ_coded = 0, differ_old = 0;
#pragma omp parallel for reduction(+ : pairs, differ, differ_coded, differ_old) schedule(dynamic, 64)
    for (int ab = 1; ab < 0x7F80; ++ab) {
      const float a = bf16((uint16_t)ab);
      const volatile float am = a > 1e-12f ? a : 1e-12f;
      const volatile float s = am / FM;
      const volatile float r = 1.0f / s;
      for (int xb = 0; xb <= ab; ++xb) {
        for (int sign = 0; sign < 2; ++sign) {
          const float x = bf16((uint16_t)(xb | (sign << 15)));
          const volatile float q0 = x * r;
          const float en = fmaf(q0, s, -x);
          const float q = fmaf(-en, r, q0);
          const float e = fmaf(-q0, s, x);
          const float q_old = copysignf(fmaf(e, r, q0), x);
          const volatile float ref = x / s;
          ++pairs;
          if (memcmp(&q, &q_old, 4) != 0) ++differ_old;
          if (memcmp(&q, (const void*)&ref, 4) != 0) {
            ++differ;
            if (fabsf(ref) >= thr || fabsf(q) >= thr) ++differ_coded;
          }
        }
      }
    }
    printf("FMAX %g pairs %lld differ %lld differ_coded %lld differ_old %lld\n", FM, pairs, differ, differ_coded, differ_old);
  }
  return 0;
}

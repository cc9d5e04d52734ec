/* Exhaustive check of the bulk quantizer's quotient sequence.
 *
 * For every fp16 value x and every positive finite fp16 max-abs a with
 * |x| <= a (the pairs a row of fp16 K or V values can hold), and both code
 * widths (qmax 127 and 7):
 *   s  = RN32(a / qmax)            the per-token scale
 *   y  = RN32(1 / s)               the correctly rounded reciprocal
 *   q0 = RN32(x * y)
 *   r  = fma(-q0, s, x)            (exact)
 *   q1 = fma(r, y, q0)
 * must equal RN32(x / s), the correctly rounded single-precision quotient
 * (IEEE division on the host). This is Markstein's correction step; the
 * program prints one summary line per code width and exits non-zero on any
 * mismatch.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float half_to_float(uint16_t h) {
  const uint32_t sign = (h >> 15) & 1u, e = (h >> 10) & 31u, m = h & 1023u;
  if (e == 0) {
    const float f = ldexpf((float)m, -24);
    return sign ? -f : f;
  }
  const uint32_t u = (sign << 31) | ((e + 112u) << 23) | (m << 13);
  float f;
  memcpy(&f, &u, 4);
  return f;
}

int main(void) {
  static float mag[0x7c00];
  int n = 0;
  for (uint32_t h = 1; h < 0x7c00; ++h) mag[n++] = half_to_float((uint16_t)h); /* positive finite, ascending */
  const float qmaxs[2] = {127.f, 7.f};
  long long total_bad = 0;
  for (int qi = 0; qi < 2; ++qi) {
    volatile float qmax = qmaxs[qi];
    long long pairs = 0, bad = 0;
    for (int ia = 0; ia < n; ++ia) {
      const float a = mag[ia];
      const float s = a / qmax;
      const float y = 1.0f / s;
      for (int ix = -1; ix <= ia; ++ix) {
        for (int neg = 0; neg < 2; ++neg) {
          const float x = ix < 0 ? 0.f : (neg ? -mag[ix] : mag[ix]);
          const float q0 = x * y;
          const float q1 = fmaf(fmaf(-q0, s, x), y, q0);
          const float ref = x / s;
          ++pairs;
          if (memcmp(&q1, &ref, 4) != 0) {
            if (bad < 5) printf("mismatch qmax=%g a=%a x=%a quotient=%a sequence=%a\n", (double)qmax, a, x, ref, q1);
            ++bad;
          }
        }
      }
    }
    printf("qmax %g: %lld pairs, %lld mismatches\n", (double)qmax, pairs, bad);
    total_bad += bad;
  }
  return total_bad ? 1 : 0;
}

/*
 * Exhaustive check of the reciprocal-based 4-bit quantiser against the IEEE
 * quotient, over the whole activation-quantisation domain: every fp16
 * amax >= 0 including +inf, with scale s = amax / 7 (fp32), and every fp16 v
 * with |v| <= amax, both signs.
 *
 *   reference : code = clamp(rint(v / s), -7, 7)   (0 when s == 0 or when the
 *               quotient is not a number)
 *   checked   : r = 1/s (0 when s == 0), q0 = v*r, e = fma(-q0, s, v),
 *               q1 = fma(e, r, q0), code = clamp(rint(q1), -7, 7), and 0 for
 *               every value of a group with an infinite scale
 *
 * Prints "pairs P quotient_mismatch Q nonzero_mismatch Z code_mismatch C";
 * Q counts pairs where q1 and v/s differ in any bit, Z those where they
 * differ other than by the sign of a zero.  Build: cc -O2 -mfma (fmaf must
 * be the fused operation; glibc's fmaf is correctly rounded either way).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float half_to_float(uint16_t h) {
  const uint32_t e = (h >> 10) & 31u, m = h & 1023u;
  const float v = e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(m | 1024u), (int)e - 25);
  return (h >> 15) ? -v : v;
}

static int clamp_rint(float q) { return (int)fminf(fmaxf(rintf(q), -7.0f), 7.0f); }

int main(void) {
  long long pairs = 0, qmis = 0, zmis = 0, cmis = 0;
  for (uint32_t ab = 0; ab <= 0x7C00u; ++ab) {
    const float amax = half_to_float((uint16_t)ab);
    const float s = amax / 7.0f;
    const float r = s == 0.0f ? 0.0f : 1.0f / s;
    for (uint32_t vb = 0; vb <= ab; ++vb) {
      for (int neg = 0; neg < 2; ++neg) {
        const float v = neg ? -half_to_float((uint16_t)vb) : half_to_float((uint16_t)vb);
        const float qref = v / s;
        const int ref = (s == 0.0f || qref != qref) ? 0 : clamp_rint(qref);
        const float q0 = v * r;
        const float e = fmaf(-q0, s, v);
        const float q1 = fmaf(e, r, q0);
        ++pairs;
        if (s != 0.0f && s < INFINITY) {
          const float q = v / s;
          uint32_t a, b;
          memcpy(&a, &q, 4);
          memcpy(&b, &q1, 4);
          if (a != b) {
            ++qmis;
            if (!(q == 0.0f && q1 == 0.0f)) ++zmis;
          }
        }
        const int code = s < INFINITY ? clamp_rint(q1) : 0;
        if (code != ref) ++cmis;
      }
    }
  }
  printf("pairs %lld quotient_mismatch %lld nonzero_mismatch %lld code_mismatch %lld\n", pairs, qmis,
         zmis, cmis);
  return cmis != 0 || zmis != 0;
}

/* The quantizer kernels compute x / d without a division per element:
 * with rd = RN(1/d), q0 = RN(x * rd), r = RN(x - q0 * d) (one fma, exact)
 * and q1 = RN(q0 + r * rd) (one fma), q1 is the correctly rounded quotient
 * (Markstein's correction).  They use it for d in [2^-60, 2^60] and
 * 0 <= x <= 2^60.  This program checks, for every non-negative finite bf16 x
 * in that range and a seeded sample of divisors (random, all-ones and
 * power-of-two significands, short significands like E4M3 scale products),
 * that q1 equals the IEEE division wherever the quotient is at least 2^-24.
 * (For x below about 2^-100 the residual r underflows and q1 can be an ulp
 * off; such quotients are below 2^-40, and every e2m1 and E4M3 code of a
 * quotient below 2^-11 is 0 whatever its last bits.)
 * Prints the counts and exits 1 on a mismatch.  Build with
 * -ffp-contract=off (no fusing beyond the explicit fmaf). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(int argc, char** argv) {
  const long nd = argc > 1 ? atol(argv[1]) : 2000;
  uint64_t s = 0x9E3779B97F4A7C15ull;
  long pairs = 0, bad = 0, low = 0;
  for (long i = 0; i < nd; ++i) {
    s ^= s << 13; s ^= s >> 7; s ^= s << 17;
    const int e = (int)(s % 121) - 60;
    uint32_t m = (uint32_t)(s >> 20) & 0x7FFFFFu;
    if (i % 4 == 1) m = 0x7FFFFFu;
    if (i % 4 == 2) m = 0;
    if (i % 4 == 3) m = (uint32_t)(s >> 40) & 0x7F0000u;
    const float d = f_of(((uint32_t)(e + 127) << 23) | m);
    const float rd = 1.0f / d;
    for (uint32_t b = 0; b <= 0x5D80u; ++b) { /* bf16 0 .. 2^60 */
      const float x = f_of(b << 16);
      const float q0 = x * rd;
      const float r = fmaf(-q0, d, x);
      const float q1 = fmaf(r, rd, q0);
      const float want = x / d;
      ++pairs;
      if (u_of(q1) != u_of(want)) {
        if (want >= 0x1p-24f || q1 >= 0x1p-24f) {
          if (bad < 5) printf("mismatch x=%a d=%a q1=%a want=%a\n", x, d, q1, want);
          ++bad;
        } else {
          ++low;
        }
      }
    }
  }
  printf("pairs %ld mismatches %ld (below 2^-24: %ld)\n", pairs, bad, low);
  return bad != 0;
}

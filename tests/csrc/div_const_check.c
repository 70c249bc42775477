/* Checks, in IEEE binary32, the correction the engine uses to divide by a
 * constant d: with c = RN(1/d), q = RN(a * c), r = RN(q * d - a) (one fused
 * multiply-add), result RN(q - r * c) (another).  For each d on the command
 * line and each binade 2^e given, every float a in [2^e, 2^(e+1)) is divided
 * both ways; the program prints "checked mismatches" for each d.  Dividing a
 * by d and scaling a by a power of two commute while a, the quotient and the
 * residual stay normal, so one binade already stands for every normal a whose
 * quotient is normal; several are checked for margin.  Build with
 * -ffp-contract=off so that a * c is rounded on its own. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static uint32_t to_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return u;
}

int main(int argc, char** argv) {
  if (argc < 3) {
    fprintf(stderr, "usage: %s d e1 [e2 ...]\n", argv[0]);
    return 2;
  }
  const float d = strtof(argv[1], NULL);
  const volatile float one = 1.0f;
  const float c = one / d;
  long long checked = 0, bad = 0;
  for (int k = 2; k < argc; ++k) {
    const int e = atoi(argv[k]);
    if (e < -126 || e > 127) return 2;
    const uint32_t base = (uint32_t)(e + 127) << 23;
    for (uint32_t m = 0; m < (1u << 23); ++m) {
      const float a = from_bits(base | m);
      const float q = a * c;
      const float r = fmaf(q, d, -a);
      const float res = fmaf(-r, c, q);
      const float ref = a / d;
      checked++;
      if (to_bits(res) != to_bits(ref)) {
        if (bad < 5) fprintf(stderr, "d=%g a=%a: %a vs %a\n", d, a, res, ref);
        bad++;
      }
    }
  }
  printf("%lld %lld\n", checked, bad);
  return 0;
}

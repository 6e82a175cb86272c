/* Host check of the fma form of the candidate step's division by 7 used by the GPU scale search:
 * q0 = RN(t * RN(1/7)), q = fma(fma(-q0, 7, t), RN(1/7), q0) must equal RN(t / 7).  Both sides
 * scale exactly with t's binade while the quotient stays normal, so the binades [1, 2) (every
 * significand), the lowest normal binades (quotients near and below the normal range) and the
 * top binade (largest quotients) cover every normal t.  Prints the number of mismatches. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static long check_binade(uint32_t e) {
  const float c = 1.0f / 7.0f;
  long bad = 0;
  for (uint32_t m = 0; m < (1u << 23); ++m) {
    const uint32_t bits = (e << 23) | m;
    float t;
    memcpy(&t, &bits, 4);
    const float ref = t / 7.0f;
    const float q0 = t * c;
    const float q = fmaf(fmaf(-q0, 7.0f, t), c, q0);
    if (q != ref) ++bad;
  }
  return bad;
}

int main(void) {
  const uint32_t binades[] = {127u, 1u, 2u, 3u, 4u, 254u};
  long bad = 0;
  for (unsigned i = 0; i < sizeof binades / sizeof binades[0]; ++i) bad += check_binade(binades[i]);
  printf("%ld\n", bad);
  return 0;
}

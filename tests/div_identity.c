/* Host check of the quantizer's scale division s = RN(M / qmax): the product
 * q0 = RN(M * RN(1/qmax)) corrected once by its exact fma remainder,
 * s = fma(fma(-q0, qmax, M), RN(1/qmax), q0), against the IEEE quotient for
 * every float M in [1, 4) (the sequence and the quotient both scale exactly by
 * powers of two away from under- and overflow).  Prints the mismatch count
 * for each divisor given on the command line. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

int main(int argc, char** argv) {
  for (int a = 1; a < argc; ++a) {
    const float b = (float)atof(argv[a]);
    volatile float one = 1.0f;
    const float r = one / b;
    long bad = 0;
    for (uint32_t u = 0x3F800000u; u < 0x40800000u; ++u) {
      const float M = from_bits(u);
      volatile float q0 = M * r;
      const float s = fmaf(fmaf(-q0, b, M), r, q0);
      volatile float t = M / b;
      if (memcmp(&s, (const void*)&t, 4) != 0) ++bad;
    }
    printf("%ld\n", bad);
  }
  return 0;
}

/* Host-side exhaustive check of the shared-reciprocal division the codec
 * kernels use, for numerators of up to 16 significant bits (bf16 / fp16
 * inputs; a device check covers every fp32 numerator). The kernels run the
 * same IEEE fp32 operations: with rh = RN(1/n), q0 = RN(a*rh), rem = fma(-q0, n, a),
 * q = fma(rem, rh, q0) must equal RN(a/n) for every numerator a with at most
 * BITS significant bits and every divisor mantissa n in [1, 2), with a in
 * [1, 2) and [2, 4) so that the quotient lies on both sides of 1. Exponent
 * shifts scale every step exactly while all values stay normal.
 *
 * usage: division_check BITS [uncorrected]
 * Prints the number of mismatches; exit status 0 iff there are none.
 * "uncorrected" checks q0 alone instead (expected to fail: it shows the
 * check can see a wrong quotient). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u) {
  float x;
  memcpy(&x, &u, sizeof x);
  return x;
}

int main(int argc, char** argv) {
  if (argc < 2) return 2;
  const int bits = atoi(argv[1]);
  const int uncorrected = argc > 2 && strcmp(argv[2], "uncorrected") == 0;
  if (bits < 1 || bits > 16) return 2;
  long long bad = 0, total = 0;
  const int nm = 1 << (bits - 1);
#pragma omp parallel for reduction(+ : bad, total) schedule(dynamic)
  for (int mx = 0; mx < nm; ++mx) {
    for (int e = 0; e < 2; ++e) {
      const float a = from_bits(((uint32_t)(127 + e) << 23) | ((uint32_t)mx << (24 - bits)));
      for (uint32_t mn = 0; mn < (1u << 23); ++mn) {
        const float n = from_bits((127u << 23) | mn);
        const float rh = 1.0f / n;
        const float q0 = a * rh;
        const float rem = fmaf(-q0, n, a);
        const float q = uncorrected ? q0 : fmaf(rem, rh, q0);
        total++;
        if (q != a / n) bad++;
      }
    }
  }
  printf("%d-bit numerators%s: %lld of %lld quotients differ\n", bits,
         uncorrected ? " (uncorrected)" : "", bad, total);
  return bad != 0;
}

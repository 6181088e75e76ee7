/* Host check of the blend kernel's seam coefficients.
 *
 * The pages (diffusers issue "[Proposal] Vectorize tiled VAE blending while
 * preserving rounding and CUDA graph replay", Proposed scope) fix the blend
 * weights as k/e and 1 - k/e computed in float64 and rounded once to fp32.
 * The kernel forms them in fp32 instead: with r = fp32(1/e) it takes
 * q0 = n * r, the exact remainder n - q0 * e by one fused multiply-add, and
 * q = q0 + rem * r by another (n = k for w_b, n = e - k for w_a).  This
 * program walks every pair 0 <= k < e <= max_e and counts the pairs where
 * that differs from the float64-rounded weight; it prints
 * "pairs P wb_mismatches B wa_mismatches A".  fmaf is C99's correctly
 * rounded fused multiply-add. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

static float corrected_quotient(float n, float e, float r) {
  const float q0 = n * r;
  const float rem = fmaf(-q0, e, n);
  return fmaf(rem, r, q0);
}

int main(int argc, char **argv) {
  const int max_e = argc > 1 ? atoi(argv[1]) : 4096;
  long pairs = 0, bad_b = 0, bad_a = 0;
  for (int e = 1; e <= max_e; ++e) {
    const float ef = (float)e;
    const float r = (float)(1.0 / (double)e);
    for (int k = 0; k < e; ++k) {
      const double q = (double)k / (double)e;
      if (corrected_quotient((float)k, ef, r) != (float)q) ++bad_b;
      if (corrected_quotient((float)(e - k), ef, r) != (float)(1.0 - q)) ++bad_a;
      ++pairs;
    }
  }
  printf("pairs %ld wb_mismatches %ld wa_mismatches %ld\n", pairs, bad_b, bad_a);
  return 0;
}

/* Host-side check of the encoder's element quotient (no GPU involved).
 *
 * The NVFP4 recipe needs q = RN(x / eff) in fp32 for every element x (a bf16 value)
 * of a block with divisor eff.  The encoder computes it from r = RN(1 / eff) as
 *     q0 = RN(x r);  e = RN(q0 eff - x);  q1 = RN(q0 - e r)
 * (the fused multiply-adds round once).  This program compares q1 with the IEEE
 * quotient x / eff for every bf16 significand of x against divisor significands
 * m = start, start + step, ... (all 2^23 of them with step 1), at exponent
 * placements whose remainder is exact (results must agree bit for bit), and at
 * placements whose remainder falls below the fp32 normal range (where q1 may miss
 * by one ulp; the E2M1 code the encoder derives from it is compared too).
 *
 * Usage: one_correction START STEP.  Prints one line per placement class and exits
 * with status 1 on a mismatch in an exact placement.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }

/* magnitude index of the E2M1 code of |q|: nearest-even on the grid
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6, saturating at 6 */
static int e2m1_index(float q) {
  static const float mid[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  const float a = fabsf(q);
  int i = 0;
  while (i < 7 && a > mid[i]) ++i;
  if (i < 7 && a == mid[i] && (i & 1)) ++i;
  return i;
}

int main(int argc, char **argv) {
  if (argc != 3) return 2;
  const uint32_t start = (uint32_t)atoi(argv[1]), step = (uint32_t)atoi(argv[2]);
  if (step == 0) return 2;
  /* exact-remainder placements (x exponent, divisor exponent) */
  static const int exact[][2] = {{0, 0}, {0, -1}, {3, 0}, {-2, 0}, {-80, -89}, {-91, -89}, {100, 97}};
  /* placements with a remainder below 2^-126 */
  static const int tiny[][2] = {{-104, -103}, {-111, -109}, {-120, -109}};
  long n_exact = 0, bad_exact = 0, n_tiny = 0, bad_tiny_q = 0, bad_tiny_code = 0;
  for (uint32_t m = start; m < (1u << 23); m += step) {
    for (int cls = 0; cls < 2; ++cls) {
      const int np = cls ? 3 : 7;
      for (int p = 0; p < np; ++p) {
        const int ex = cls ? tiny[p][0] : exact[p][0], eb = cls ? tiny[p][1] : exact[p][1];
        const float b = ldexpf(from_bits(0x3F800000u | m), eb);
        const float r = 1.0f / b;
        for (uint32_t s = 0; s < 128; ++s) {
          const float x = ldexpf(from_bits(0x3F800000u | (s << 16)), ex);
          if (bits(x) & 0xFFFFu) continue; /* not a bf16 value at this exponent */
          const float want = x / b;
          const float q0 = x * r;
          const float e = fmaf(q0, b, -x);
          const float q1 = fmaf(-e, r, q0);
          if (cls == 0) {
            ++n_exact;
            if (bits(q1) != bits(want)) {
              if (++bad_exact <= 5) printf("mismatch x=%a eff=%a want=%a got=%a\n", x, b, want, q1);
            }
          } else {
            ++n_tiny;
            if (bits(q1) != bits(want)) ++bad_tiny_q;
            if (e2m1_index(q1) != e2m1_index(want)) ++bad_tiny_code;
          }
        }
      }
    }
  }
  printf("exact remainder: %ld quotients, %ld mismatches\n", n_exact, bad_exact);
  printf("remainder below the normal range: %ld quotients, %ld off by an ulp, %ld with another code\n", n_tiny,
         bad_tiny_q, bad_tiny_code);
  return bad_exact ? 1 : 0;
}

/* The append's scale byte starts from RN(amax / 6).  One code path forms it with
   two Markstein corrections from r = RN(1/6) (amax >= 2^-90), another with an IEEE
   division; this program checks that the two agree for every finite non-negative
   bf16 magnitude at or above 2^-90 (and for zero), using the host's fp32
   arithmetic with fused multiply-add (compiled without contraction). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* q0 = RN(x r), then two corrections with the negated remainder q b - x */
static float two_corrections(float x, float b, float r) {
  float q = x * r;
  float e = fmaf(q, b, -x);
  q = fmaf(-e, r, q);
  e = fmaf(q, b, -x);
  return fmaf(-e, r, q);
}

int main(void) {
  const float six = 6.0f, r = 1.0f / six, lo = ldexpf(1.0f, -90);
  long checked = 0, bad = 0;
  for (uint32_t h = 0; h < 0x7F80u; ++h) {          /* +0 up to the largest finite bf16 */
    const float x = from_bits(h << 16);
    if (!(x == 0.0f || x >= lo)) continue;
    const float a = two_corrections(x, six, r), b = x / six;
    ++checked;
    if (to_bits(a) != to_bits(b)) {
      if (bad < 10) printf("mismatch: x = %a: corrected %a, IEEE %a\n", x, a, b);
      ++bad;
    }
  }
  printf("%ld magnitudes checked, %ld mismatches\n", checked, bad);
  return bad != 0;
}

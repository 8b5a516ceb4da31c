/* The library's E4M3FN encoder is branch-free: with e = max(exponent of |v|, -6), the code is
 * (e + 7) * 8 - 8 + rint(|v| * 2^(3 - e)), at most 126 (448), NaN -> 0x7F, sign bit 0x80.
 * This program restates that form in C (binary32, no contraction) and compares it with an
 * encoder written from the E4M3FN definition (4 exponent bits, bias 7, 3 fraction bits,
 * subnormals spaced 2^-9, largest finite 448; nearest code, ties to the even code, saturated)
 * on every Nth binary32 pattern and on every pattern of the binades on either side of 2^-6
 * (the subnormal/normal edge) and of [256, 512) (saturation at 448).
 * Usage: e4m3_encoder N  -> prints the counts, exit status 1 on any mismatch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* value of the non-negative code k (0..126) */
static double e4m3_value(int k) {
  const int e = k >> 3, f = k & 7;
  return e == 0 ? ldexp((double)f, -9) : ldexp(1.0 + f / 8.0, e - 7);
}
/* nearest code to |v| (ties to the even code), saturated at 448 = code 126; the sign bit
 * of v gives 0x80, so -0 and negative values that round to zero give 0x80 */
static unsigned encode(float v) {
  const unsigned sign = signbit(v) ? 0x80u : 0u;
  const double a = fabs((double)v);
  if (a >= 448.0) return sign | 126u;
  int lo = 0, hi = 126;  /* largest code with value <= a */
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (e4m3_value(mid) <= a) lo = mid; else hi = mid - 1;
  }
  if (lo == 126) return sign | 126u;
  const double d0 = a - e4m3_value(lo), d1 = e4m3_value(lo + 1) - a;
  const int k = (d0 < d1) ? lo : (d1 < d0) ? lo + 1 : ((lo & 1) ? lo + 1 : lo);
  return sign | (unsigned)k;
}

static unsigned closed_form(float v) {
  uint32_t u;
  memcpy(&u, &v, 4);
  const float ax = fabsf(v);
  int e = (int)((u >> 23) & 0xFFu) - 127;
  if (e < -6) e = -6;
  const float code = fminf((float)((e + 7) * 8 - 8) + rintf(ldexpf(ax, 3 - e)), 126.0f);
  return (ax == ax) ? (((u >> 24) & 0x80u) | (unsigned)code) : 0x7Fu;
}
int main(int argc, char **argv) {
  const long stride = argc > 1 ? atol(argv[1]) : 61;
  long n = 0, bad = 0;
  for (uint64_t i = 0; i < (1ull << 32); i += (uint64_t)stride) {
    const uint32_t u = (uint32_t)i;
    float v;
    memcpy(&v, &u, 4);
    const unsigned want = (v == v) ? encode(v) : 0x7Fu;
    bad += closed_form(v) != want;
    ++n;
  }
  /* binades [2^-7, 2^-5) and [256, 512), both signs, every pattern */
  const uint32_t lo[2] = {(127u - 7u) << 23, (127u + 8u) << 23}, hi[2] = {(127u - 5u) << 23, (127u + 9u) << 23};
  for (int r = 0; r < 2; ++r)
    for (uint32_t u = lo[r]; u < hi[r]; ++u)
      for (uint32_t sg = 0; sg < 2; ++sg) {
        const uint32_t w = u | (sg << 31);
        float v;
        memcpy(&v, &w, 4);
        bad += closed_form(v) != encode(v);
        ++n;
      }
  /* signed zeros, infinities, the smallest binary32 subnormals, NaNs, the tie 2^-10 between
   * codes 0 and 1 (to 0, even), just above it, and 2^-9 (code 1) */
  const uint32_t special[] = {0x00000000u, 0x80000000u, 0x7F800000u, 0xFF800000u, 0x00000001u, 0x80000001u,
                              0x7FC00000u, 0xFFC00001u, 0x3A800000u, 0xBA800000u, 0x3A800001u, 0x3B000000u};
  const unsigned expect[] = {0x00, 0x80, 0x7E, 0xFE, 0x00, 0x80, 0x7F, 0x7F, 0x00, 0x80, 0x01, 0x01};
  for (int k = 0; k < (int)(sizeof special / sizeof special[0]); ++k) {
    float v;
    memcpy(&v, &special[k], 4);
    bad += closed_form(v) != expect[k];
    ++n;
  }
  printf("encoder patterns %ld mismatches %ld\n", n, bad);
  return (bad || n == 0) ? 1 : 0;
}

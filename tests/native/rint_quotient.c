/* The bulk append's quantizer takes rint(fl(x / s)) without one division per value:
 * q0 = fl(x * fl(1/s)) is within 2^-16 of x/s when |x/s| <= lim (1 + 2^-11) < 128, so
 * rint(q0) equals rint(fl(x/s)) unless q0 lies within 2^-15 of a half-integer (where the
 * kernel divides exactly).  This program restates that rule in C (IEEE binary32, no
 * contraction) and compares it with the division for fp16 scales across their whole range
 * (subnormals included), values spread over the code range, and values a few ulps around
 * every rounding boundary (k + 1/2) * s.  It also checks the rule when the product and the
 * subtraction are fused into one fma, as a compiler may contract them.
 * Usage: rint_quotient N  -> prints the counts, exit status 1 on any mismatch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) {
  st ^= st << 13;
  st ^= st >> 7;
  st ^= st << 17;
  return st;
}
static float f16_value(uint16_t h) { /* exact, positive */
  const int e = (h >> 10) & 31, m = h & 1023;
  return e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(m | 1024), e - 25);
}

int main(int argc, char **argv) {
  const long iters = argc > 1 ? atol(argv[1]) : 10000000L;
  long n = 0, amb = 0, bad = 0, bad_fused = 0;
  for (long it = 0; it < iters; ++it) {
    const uint16_t h = (uint16_t)(1 + next() % 0x7BFF); /* finite positive fp16 */
    volatile float s = f16_value(h);
    volatile float rs = 1.0f / s;
    const int lim = (it & 1) ? 127 : 7; /* INT8 and 4-bit codes */
    const uint64_t r = next();
    float x;
    if (r & 1) { /* a few ulps around the boundary (k + 1/2) s, which is exact in binary32 */
      const int k = (int)((r >> 1) % (uint64_t)(2 * lim + 1)) - lim;
      volatile float b = ((float)k + 0.5f) * s;
      int32_t bits;
      memcpy(&bits, (const void *)&b, 4);
      bits += (int32_t)((r >> 20) % 9) - 4;
      memcpy(&x, &bits, 4);
    } else {
      x = ((float)(int32_t)(r >> 32) / 2147483648.0f) * (float)lim * s;
    }
    if (!(fabsf(x / s) <= (float)lim * (1.0f + 0x1p-11f))) continue;
    ++n;
    volatile float q0 = x * rs;
    const float n0 = rintf(q0);
    const float exact = rintf(x / s);
    if (0.5f - fabsf(q0 - n0) <= 0x1p-15f)
      ++amb;
    else if (n0 != exact)
      ++bad;
    if (!(0.5f - fabsf(fmaf(x, rs, -n0)) <= 0x1p-15f) && n0 != exact) ++bad_fused;
  }
  printf("cases %ld near a boundary %ld mismatches %ld (fused %ld)\n", n, amb, bad, bad_fused);
  return (bad || bad_fused || n == 0) ? 1 : 0;
}

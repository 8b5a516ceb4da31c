/*
 * kvq_oracle.c -- plain, slow, obviously correct CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py; never by the HIP library.  Shares no code with
 * it.  Built with gcc -O2 -ffp-contract=off (no fast-math) so every float
 * operation below is one IEEE-754 binary32 or binary64 operation.
 *
 * Quantization runs in fp32 (the precision in which the codes are decided);
 * attention runs in fp64.
 */
#include "kvq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

/* IEEE binary16 from binary32, round to nearest, ties to even.  binary16 has
 * 1 sign bit, 5 exponent bits (bias 15) and 10 fraction bits; subnormals are
 * multiples of 2^-24; the largest finite value is 65504. */
uint16_t orc_f32_to_f16_rne(float f) {
  uint32_t x = f32_bits(f);
  uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
  uint32_t ax = x & 0x7FFFFFFFu;
  if (ax > 0x7F800000u) return (uint16_t)(sign | 0x7E00u); /* NaN stays NaN */
  /* 65520 = 65504 + half an ulp: the tie rounds to the even neighbour 2^16,
   * which overflows to infinity; anything at or above it does too. */
  if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u);
  int e = (int)(ax >> 23) - 127; /* unbiased exponent of a normal binary32 */
  if (e >= -14) {
    /* normal binary16: keep the top 10 fraction bits, round on the other 13 */
    uint32_t frac = ax & 0x7FFFFFu;
    uint32_t h = ((uint32_t)(e + 15) << 10) | (frac >> 13);
    uint32_t rest = frac & 0x1FFFu;
    if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) h += 1u; /* carry may bump exponent: correct */
    return (uint16_t)(sign | h);
  }
  /* subnormal binary16 or zero: result = round(|f| / 2^-24) */
  if (e < -25) return sign; /* |f| < 2^-25: below half the smallest subnormal */
  uint32_t sig = (ax & 0x7FFFFFu) | 0x800000u; /* |f| = sig * 2^(e-23) */
  int shift = -e - 1;                          /* |f| / 2^-24 = sig * 2^(e+1) */
  uint32_t m = sig >> shift;
  uint32_t rest = sig & ((1u << shift) - 1u);
  uint32_t half = 1u << (shift - 1);
  if (rest > half || (rest == half && (m & 1u))) m += 1u; /* m == 1024 encodes 2^-14 */
  return (uint16_t)(sign | m);
}

float orc_f16_to_f32(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  return (float)(s ? -v : v);
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
float orc_bf16_to_f32(uint16_t b) {
  int s = (b >> 15) & 1, e = (b >> 7) & 255, m = b & 127;
  double v;
  if (e == 0)
    v = ldexp((double)m, -133); /* m/128 * 2^-126 */
  else if (e == 255)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(128 + m), e - 134); /* (1 + m/128) * 2^(e-127) */
  return (float)(s ? -v : v);
}

/* bfloat16 from binary32: keep the top 16 bits, rounding the lower 16 to nearest, ties
 * to even (a carry may bump the exponent, up to infinity); NaN gives a quiet NaN. */
uint16_t orc_f32_to_bf16_rne(float f) {
  uint32_t x = f32_bits(f);
  if ((x & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((x >> 16) | 0x0040u);
  uint32_t hi = x >> 16, rest = x & 0xFFFFu;
  if (rest > 0x8000u || (rest == 0x8000u && (hi & 1u))) hi += 1u;
  return (uint16_t)hi;
}

/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 fraction bits, no
 * infinities; S.1111.111 is NaN; subnormals are multiples of 2^-9; the
 * largest finite magnitude is 448 (code 0x7E). */
float orc_e4m3fn_to_f32(uint8_t c) {
  int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return (float)(s ? -v : v);
}

/* The 127 finite non-negative E4M3FN magnitudes, ascending with the code. */
static double g_e4m3_mag[127];
static int g_e4m3_ready = 0;

static void e4m3_table(void) {
  if (g_e4m3_ready) return;
  for (int c = 0; c < 127; ++c) g_e4m3_mag[c] = (double)orc_e4m3fn_to_f32((uint8_t)c);
  g_e4m3_ready = 1;
}

/* Nearest representable magnitude, ties to the even code (= even fraction
 * LSB); magnitudes beyond 448 take 448 (saturation to the largest finite
 * value); the sign is kept, so negative values that round to zero give 0x80. */
uint8_t orc_f32_to_e4m3fn(float f) {
  e4m3_table();
  if (isnan(f)) return 0x7F;
  uint8_t sign = signbit(f) ? 0x80 : 0x00;
  double a = fabs((double)f);
  /* binary search: first code whose magnitude is >= a */
  int lo = 0, hi = 126;
  if (a >= g_e4m3_mag[126]) return (uint8_t)(sign | 126);
  while (lo < hi) {
    int mid = (lo + hi) / 2;
    if (g_e4m3_mag[mid] >= a)
      hi = mid;
    else
      lo = mid + 1;
  }
  int up = lo; /* g_e4m3_mag[up] >= a */
  if (up == 0) return sign;
  int dn = up - 1;
  double du = g_e4m3_mag[up] - a, dd = a - g_e4m3_mag[dn]; /* exact in binary64 */
  int pick;
  if (du < dd)
    pick = up;
  else if (dd < du)
    pick = dn;
  else
    pick = (up % 2 == 0) ? up : dn;
  return (uint8_t)(sign | pick);
}

/* ------------------------------------------------------------------------ */
/* Quantizers                                                                */
/* ------------------------------------------------------------------------ */

/* Per 64-dim group: a = max|x|; s = fp16(a / 127) (fp32 division, RNE to
 * fp16: this is the stored scale); c = clamp(rint(x / s), -127, 127) with the
 * stored scale widened to fp32; s == 0 gives all-zero codes. */
void orc_quant_int8_g64(const float *x, int D, int8_t *codes, uint16_t *scales) {
  for (int g = 0; g < D / 64; ++g) {
    const float *xg = x + 64 * g;
    float a = 0.0f;
    for (int i = 0; i < 64; ++i) {
      float v = fabsf(xg[i]);
      if (v > a) a = v;
    }
    float s32 = a / 127.0f;
    uint16_t h = orc_f32_to_f16_rne(s32);
    float s = orc_f16_to_f32(h);
    scales[g] = h;
    for (int i = 0; i < 64; ++i) {
      int c = 0;
      if (s != 0.0f) {
        float r = rintf(xg[i] / s);
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        c = (int)r;
      }
      codes[64 * g + i] = (int8_t)c;
    }
  }
}

/* Per row: a = max|x|; s = a / 448 in fp32 (stored); code = E4M3FN(x / s);
 * s == 0 gives all-zero codes. */
void orc_quant_fp8_row(const float *x, int D, uint8_t *codes, float *scale) {
  float a = 0.0f;
  for (int i = 0; i < D; ++i) {
    float v = fabsf(x[i]);
    if (v > a) a = v;
  }
  float s = a / 448.0f;
  *scale = s;
  for (int i = 0; i < D; ++i) codes[i] = (s != 0.0f) ? orc_f32_to_e4m3fn(x[i] / s) : 0;
}

/* RotorQuant rk8v4 keys.  The 64-point Hadamard matrix in Sylvester order has
 * entry (-1)^popcount(i & j) at row j, column i; divided by 8 = sqrt(64) it is
 * orthonormal and its own inverse.  The sum runs in binary64 in index order: for
 * bf16 sources (8 significant bits) it is exact unless the 64 magnitudes span more
 * than 2^39, so the single rounding to binary32 gives the correctly rounded rotation. */
void orc_h64_rotate(const float *x, float *y) {
  for (int j = 0; j < 64; ++j) {
    double acc = 0.0;
    for (int i = 0; i < 64; ++i) {
      int odd = __builtin_popcount((unsigned)(i & j)) & 1;
      acc += odd ? -(double)x[i] : (double)x[i];
    }
    y[j] = (float)(acc / 8.0);
  }
}

/* Rotate each 64-dim group, then the INT8 group-64 encoding of the rotated row. */
void orc_quant_rk8v4_k(const float *x, int D, int8_t *codes, uint16_t *scales) {
  float *y = (float *)malloc(sizeof(float) * D);
  for (int g = 0; g < D / 64; ++g) orc_h64_rotate(x + 64 * g, y + 64 * g);
  orc_quant_int8_g64(y, D, codes, scales);
  free(y);
}

/* rk4v4 keys.  Lloyd's iteration for the minimum-mean-square-error quantizer of a
 * standard Gaussian with 16 levels: each threshold is the midpoint of its two
 * neighbouring levels, each level the mean of N(0,1) over its cell,
 * E[X | a < X <= b] = (phi(a) - phi(b)) / (Phi(b) - Phi(a)).  Started from evenly
 * spaced levels and run until no level moves (binary64). */
static double std_pdf(double x) { return isinf(x) ? 0.0 : exp(-0.5 * x * x) / sqrt(2.0 * acos(-1.0)); }
static double std_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

void orc_lloyd_max16(double *L) {
  for (int i = 0; i < 16; ++i) L[i] = -3.0 + 6.0 * i / 15.0;
  for (int it = 0; it < 100000; ++it) {
    double t[17], nl[16], moved = 0.0;
    t[0] = -INFINITY;
    t[16] = INFINITY;
    for (int i = 1; i < 16; ++i) t[i] = 0.5 * (L[i - 1] + L[i]);
    for (int i = 0; i < 16; ++i) {
      nl[i] = (std_pdf(t[i]) - std_pdf(t[i + 1])) / (std_cdf(t[i + 1]) - std_cdf(t[i]));
      moved = fmax(moved, fabs(nl[i] - L[i]));
    }
    for (int i = 0; i < 16; ++i) L[i] = nl[i];
    if (moved < 1e-15) break;
  }
}

void orc_rk4_codes(int8_t *codes) {
  double L[16];
  orc_lloyd_max16(L);
  for (int i = 0; i < 16; ++i) codes[i] = (int8_t)rint(127.0 * L[i] / L[15]);
}

static int8_t g_rk4_code[16];
static int g_rk4_ready = 0;
static const int8_t *rk4_codes(void) {
  if (!g_rk4_ready) {
    orc_rk4_codes(g_rk4_code);
    g_rk4_ready = 1;
  }
  return g_rk4_code;
}

/* Rotate each 64-dim group; per group a = max|y|, s = fp16(a / 127) (the INT8 scale);
 * u = y / s in fp32; the index is the number of level midpoints (c_i + c_{i+1}) / 2
 * strictly below u, i.e. the level whose code is nearest to u, ties to the lower one.
 * s == 0 gives u = 0 for every element. */
void orc_quant_rk4v4_k(const float *x, int D, uint8_t *idx, uint16_t *scales) {
  const int8_t *c = rk4_codes();
  float *y = (float *)malloc(sizeof(float) * D);
  for (int g = 0; g < D / 64; ++g) orc_h64_rotate(x + 64 * g, y + 64 * g);
  for (int g = 0; g < D / 64; ++g) {
    const float *yg = y + 64 * g;
    float a = 0.0f;
    for (int i = 0; i < 64; ++i) {
      float v = fabsf(yg[i]);
      if (v > a) a = v;
    }
    uint16_t h = orc_f32_to_f16_rne(a / 127.0f);
    float sc = orc_f16_to_f32(h);
    scales[g] = h;
    for (int i = 0; i < 64; ++i) {
      float u = (sc != 0.0f) ? yg[i] / sc : 0.0f;
      int k = 0;
      for (int m = 0; m < 15; ++m)
        if (0.5f * (float)(c[m] + c[m + 1]) < u) ++k;
      idx[64 * g + i] = (uint8_t)k;
    }
  }
  free(y);
}

/* Per 32-dim group: a = max|x|; s = fp16(a / 7) (fp32 division, RNE to fp16);
 * c = clamp(rint(x / s), -7, 7) with the stored scale widened to fp32; s == 0
 * gives all-zero codes.  Four bits hold the 15 levels -7..7. */
void orc_quant_int4_g32(const float *x, int D, int8_t *codes, uint16_t *scales) {
  for (int g = 0; g < D / 32; ++g) {
    const float *xg = x + 32 * g;
    float a = 0.0f;
    for (int i = 0; i < 32; ++i) {
      float v = fabsf(xg[i]);
      if (v > a) a = v;
    }
    uint16_t h = orc_f32_to_f16_rne(a / 7.0f);
    float step = orc_f16_to_f32(h);
    scales[g] = h;
    for (int i = 0; i < 32; ++i) {
      int c = 0;
      if (step != 0.0f) {
        float q = rintf(xg[i] / step);
        if (q > 7.0f) q = 7.0f;
        if (q < -7.0f) q = -7.0f;
        c = (int)q;
      }
      codes[32 * g + i] = (int8_t)c;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Page layout (one page = 64 token slots of one KV head in one block)       */
/* ------------------------------------------------------------------------ */

/* K: 16x16-byte tiles; tile (s/16, d/16) holds 16 slots x 16 dims, slot-major;
 * tiles ordered slot-group-major. */
int64_t orc_k_byte(int s, int d, int D) {
  return ((int64_t)(s / 16) * (D / 16) + d / 16) * 256 + (s % 16) * 16 + (d % 16);
}

/* V: dim-major.  For dim d, the 64 slots sit in four 16-byte runs; run
 * r = (s % 16) / 4 holds the slots 16*j + 4*r + i (j, i in 0..3) at byte 4*j + i.
 * Runs are ordered (d / 16, r, d % 16). */
int64_t orc_v_byte(int s, int d, int D) {
  (void)D;
  int r = (s % 16) / 4;
  return ((int64_t)(d / 16) * 4 + r) * 256 + (d % 16) * 16 + (s / 16) * 4 + (s % 4);
}

/* rk8v4 V: 4-bit codes, 64*D/2 bytes per page.  The 16 slots of run r of dim d
 * take 8 bytes, two 32-bit little-endian words: word w holds the slots
 * 16*j + 4*r + i with j in {2w, 2w+1}; with k = 4*(j % 2) + i, the code of k sits
 * at bit 16*(k % 2) + 4*(k / 2) of the word (codes k, k+1 in the two 16-bit halves).
 * The 8-byte chunks are ordered (d/32, r, d%16, (d/16)%2): the two 16-dim tiles
 * of a 32-dim pair sit side by side. */
int64_t orc_v4_bit(int s, int d, int D) {
  (void)D;
  int r = (s % 16) / 4, j = s / 16, i = s % 4;
  int dt = d / 16;
  int64_t word = (((int64_t)(dt / 2) * 64 + r * 16 + d % 16) * 16 + (dt % 2) * 8 + (j / 2) * 4);
  int k = (j % 2) * 4 + i;
  return word * 8 + 16 * (k % 2) + 4 * (k / 2);
}

/* rk4v4 K: 4-bit level indices, 64*D/2 bytes per page.  The 16 dims 16*(d/16) .. +15
 * of slot s take 8 bytes: two 32-bit words (dims 0..7 and 8..15 of the 16), whose
 * byte b holds dim b (low nibble) and dim b + 4 (high nibble) of its 8.  The 8-byte
 * chunks of the two 64-dim groups 2p, 2p+1 sit side by side, and the 16-byte units
 * are ordered (s/16, d/128, (d%64)/16, s%16). */
int64_t orc_k4_bit(int s, int d, int D) {
  int64_t unit = ((int64_t)(s / 16) * (D / 128) + d / 128) * 64 + ((d % 64) / 16) * 16 + (s % 16);
  int64_t byte = unit * 16 + ((d / 64) % 2) * 8 + ((d % 16) / 8) * 4 + (d % 4);
  return byte * 8 + 4 * ((d % 8) / 4);
}

/* Scales follow the same slot runs: run r = (s % 16) / 4 is the slowest index.
 * INT8 (and rk8v4) K scales: (run, s/16, group, s%4); INT8 V scales: (run, group, s/16, s%4);
 * rk8v4 V scales: (run, 32-dim group, s/16, s%4); FP8 scales (K and V): (run, s/16, s%4). */
int64_t orc_scale_elem(int fmt, int which, int s, int g, int D) {
  int r = (s % 16) / 4, j = s / 16, i = s % 4;
  if (fmt == ORC_FMT_INT8_G64 || ((fmt == ORC_FMT_RK8V4 || fmt == ORC_FMT_RK4V4) && which == 0)) {
    if (which == 0) return (((int64_t)r * 4 + j) * (D / 64) + g) * 4 + i;
    return ((int64_t)r * (D / 64) + g) * 16 + j * 4 + i;
  }
  if (fmt == ORC_FMT_RK8V4 || fmt == ORC_FMT_RK4V4) return ((int64_t)r * (D / 32) + g) * 16 + j * 4 + i;
  return (int64_t)r * 16 + j * 4 + i;
}

static int64_t page_index(const orc_pool *p, int block, int kvh) {
  return (int64_t)block * p->num_kv_heads + kvh;
}

static float load_src(const void *src, int dtype, int64_t i) {
  if (dtype == ORC_SRC_BF16) return orc_bf16_to_f32(((const uint16_t *)src)[i]);
  return ((const float *)src)[i];
}

int orc_append(const orc_pool *p, const void *k_new, const void *v_new, int src_dtype, int B,
               int n_new, const int32_t *block_table, int max_blocks, const int32_t *start_pos) {
  const int H = p->num_kv_heads, D = p->head_dim, G = D / 64;
  float *x = (float *)malloc(sizeof(float) * D);
  uint8_t *codes = (uint8_t *)malloc(D);
  uint16_t *s16 = (uint16_t *)malloc(sizeof(uint16_t) * (D / 32 > 0 ? D / 32 : 1));
  int rc = 0;
  for (int b = 0; b < B && rc == 0; ++b) {
    for (int t = 0; t < n_new && rc == 0; ++t) {
      int64_t pos = (int64_t)start_pos[b] + t;
      if (pos < 0 || pos / 64 >= max_blocks) {
        rc = -1;
        break;
      }
      int block = block_table[(int64_t)b * max_blocks + pos / 64];
      int slot = (int)(pos % 64);
      if (block < 0 || block >= p->num_blocks) {
        rc = -1;
        break;
      }
      for (int which = 0; which < 2; ++which) {
        const void *src = which ? v_new : k_new;
        uint8_t *pool_codes = which ? p->v_codes : p->k_codes;
        void *pool_scales = which ? p->v_scales : p->k_scales;
        for (int h = 0; h < H; ++h) {
          int64_t row = (((int64_t)b * n_new + t) * H + h) * D;
          for (int d = 0; d < D; ++d) x[d] = load_src(src, src_dtype, row + d);
          int64_t pg = page_index(p, block, h);
          if (p->format == ORC_FMT_BF16) {
            uint16_t *page16 = (uint16_t *)pool_codes + pg * 64 * D;
            for (int d = 0; d < D; ++d)
              page16[which ? orc_v_byte(slot, d, D) : orc_k_byte(slot, d, D)] = orc_f32_to_bf16_rne(x[d]);
            continue;
          }
          if ((p->format == ORC_FMT_RK8V4 || p->format == ORC_FMT_RK4V4) && which == 1) {
            uint8_t *page4 = pool_codes + pg * 64 * (D / 2);
            orc_quant_int4_g32(x, D, (int8_t *)codes, s16);
            uint16_t *sc = (uint16_t *)pool_scales + pg * 64 * (D / 32);
            for (int g = 0; g < D / 32; ++g) sc[orc_scale_elem(p->format, which, slot, g, D)] = s16[g];
            for (int d = 0; d < D; ++d) {
              int64_t bit = orc_v4_bit(slot, d, D);
              uint8_t nib = (uint8_t)(codes[d] & 0x0F); /* two's complement nibble */
              uint8_t *byte = page4 + bit / 8;
              int sh = (int)(bit % 8);
              *byte = (uint8_t)((*byte & ~(0x0F << sh)) | (nib << sh));
            }
            continue;
          }
          if (p->format == ORC_FMT_RK4V4) {
            uint8_t *page4 = pool_codes + pg * 64 * (D / 2);
            orc_quant_rk4v4_k(x, D, codes, s16);
            uint16_t *sc = (uint16_t *)pool_scales + pg * 64 * G;
            for (int g = 0; g < G; ++g) sc[orc_scale_elem(p->format, which, slot, g, D)] = s16[g];
            for (int d = 0; d < D; ++d) {
              int64_t bit = orc_k4_bit(slot, d, D);
              uint8_t *byte = page4 + bit / 8;
              int sh = (int)(bit % 8);
              *byte = (uint8_t)((*byte & ~(0x0F << sh)) | ((codes[d] & 0x0F) << sh));
            }
            continue;
          }
          uint8_t *page = pool_codes + pg * 64 * D;
          if (p->format == ORC_FMT_RK8V4) {
            orc_quant_rk8v4_k(x, D, (int8_t *)codes, s16);
            uint16_t *sc = (uint16_t *)pool_scales + pg * 64 * G;
            for (int g = 0; g < G; ++g) sc[orc_scale_elem(p->format, which, slot, g, D)] = s16[g];
          } else if (p->format == ORC_FMT_INT8_G64) {
            orc_quant_int8_g64(x, D, (int8_t *)codes, s16);
            uint16_t *sc = (uint16_t *)pool_scales + pg * 64 * G;
            for (int g = 0; g < G; ++g) sc[orc_scale_elem(p->format, which, slot, g, D)] = s16[g];
          } else {
            float s;
            orc_quant_fp8_row(x, D, codes, &s);
            float *sc = (float *)pool_scales + pg * 64;
            sc[orc_scale_elem(p->format, which, slot, 0, D)] = s;
          }
          for (int d = 0; d < D; ++d)
            page[which ? orc_v_byte(slot, d, D) : orc_k_byte(slot, d, D)] = codes[d];
        }
      }
    }
  }
  free(x);
  free(codes);
  free(s16);
  return rc;
}

/* Dequantized value: code * scale, exact in binary64.  rk8v4 keys stay in the
 * rotated domain; rk8v4 values are the sign-extended nibble times its group scale. */
double orc_dequant(const orc_pool *p, int which, int block, int kvh, int slot, int d) {
  const int D = p->head_dim;
  int64_t pg = page_index(p, block, kvh);
  if (p->format == ORC_FMT_BF16) {
    const uint16_t *page16 = (const uint16_t *)(which ? p->v_codes : p->k_codes) + pg * 64 * D;
    return (double)orc_bf16_to_f32(page16[which ? orc_v_byte(slot, d, D) : orc_k_byte(slot, d, D)]);
  }
  if (p->format == ORC_FMT_RK4V4 && which == 0) {
    const uint8_t *page4 = p->k_codes + pg * 64 * (D / 2);
    int64_t bit = orc_k4_bit(slot, d, D);
    int nib = (page4[bit / 8] >> (bit % 8)) & 0x0F;
    uint16_t h = ((const uint16_t *)p->k_scales)[pg * 64 * (D / 64) + orc_scale_elem(p->format, 0, slot, d / 64, D)];
    return (double)rk4_codes()[nib] * (double)orc_f16_to_f32(h);
  }
  if ((p->format == ORC_FMT_RK8V4 || p->format == ORC_FMT_RK4V4) && which == 1) {
    const uint8_t *page4 = p->v_codes + pg * 64 * (D / 2);
    int64_t bit = orc_v4_bit(slot, d, D);
    int nib = (page4[bit / 8] >> (bit % 8)) & 0x0F;
    int c = nib >= 8 ? nib - 16 : nib;
    uint16_t h = ((const uint16_t *)p->v_scales)[pg * 64 * (D / 32) + orc_scale_elem(p->format, 1, slot, d / 32, D)];
    return (double)c * (double)orc_f16_to_f32(h);
  }
  const uint8_t *page = (which ? p->v_codes : p->k_codes) + pg * 64 * D;
  uint8_t byte = page[which ? orc_v_byte(slot, d, D) : orc_k_byte(slot, d, D)];
  const void *scales = which ? p->v_scales : p->k_scales;
  if (p->format == ORC_FMT_INT8_G64 || p->format == ORC_FMT_RK8V4) {
    uint16_t h = ((const uint16_t *)scales)[pg * 64 * (D / 64) + orc_scale_elem(p->format, which, slot, d / 64, D)];
    return (double)(int8_t)byte * (double)orc_f16_to_f32(h);
  }
  float s = ((const float *)scales)[pg * 64 + orc_scale_elem(p->format, which, slot, 0, D)];
  return (double)orc_e4m3fn_to_f32(byte) * (double)s;
}

/* ------------------------------------------------------------------------ */
/* Attention                                                                 */
/* ------------------------------------------------------------------------ */

/* out[r] = sum_j w_j v_j / sum_j w_j with w_j = exp(z_j - max z),
 * z_j = scale * <q_r, k_j>, over j = 0..last[r]. */
int orc_dense_attn(const double *q, const double *k, const double *v, int nq, int L, int D,
                   double scale, const int32_t *last, double *out) {
  double *z = (double *)malloc(sizeof(double) * (L > 0 ? L : 1));
  for (int r = 0; r < nq; ++r) {
    int n = last[r] + 1;
    if (n < 1 || n > L) {
      free(z);
      return -1;
    }
    const double *qr = q + (int64_t)r * D;
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
      double acc = 0.0;
      for (int d = 0; d < D; ++d) acc += qr[d] * k[(int64_t)j * D + d];
      z[j] = scale * acc;
      if (z[j] > m) m = z[j];
    }
    double l = 0.0;
    double *o = out + (int64_t)r * D;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    for (int j = 0; j < n; ++j) {
      double w = exp(z[j] - m);
      l += w;
      for (int d = 0; d < D; ++d) o[d] += w * v[(int64_t)j * D + d];
    }
    for (int d = 0; d < D; ++d) o[d] /= l;
  }
  free(z);
  return 0;
}

/* The same definition over the paged pool: key j of sequence b is slot j % 64
 * of block block_table[b][j / 64]; K and V are dequantized on the way. */
int orc_paged_attn(const orc_pool *p, const void *q, int q_dtype, int B, int T, int Hq,
                   const int32_t *block_table, int max_blocks, const int32_t *seq_lens,
                   float softmax_scale, const int32_t *rows, int nrows, double *out) {
  const int D = p->head_dim, Hkv = p->num_kv_heads;
  if (Hkv <= 0 || Hq % Hkv != 0) return -1;
  const int G = Hq / Hkv;
  const int total = B * T * Hq;
  const int n = rows ? nrows : total;
  int Lmax = 0;
  for (int b = 0; b < B; ++b)
    if (seq_lens[b] > Lmax) Lmax = seq_lens[b];
  double *z = (double *)malloc(sizeof(double) * (Lmax > 0 ? Lmax : 1));
  double *qd = (double *)malloc(sizeof(double) * D);
  double *row = (double *)malloc(sizeof(double) * D);
  int rc = 0;
  for (int i = 0; i < n && rc == 0; ++i) {
    int flat = rows ? rows[i] : i;
    if (flat < 0 || flat >= total) {
      rc = -1;
      break;
    }
    int h = flat % Hq, t = (flat / Hq) % T, b = flat / (Hq * T);
    int kvh = h / G;
    int last = seq_lens[b] - T + t;
    if (last < 0 || (last / 64) >= max_blocks) {
      rc = -1;
      break;
    }
    for (int d = 0; d < D; ++d) qd[d] = (double)load_src(q, q_dtype, (int64_t)flat * D + d);
    if (p->format == ORC_FMT_RK8V4 || p->format == ORC_FMT_RK4V4) {
      /* the keys are stored rotated: rotate the query by the same orthonormal
       * matrix (in binary64), so that <H q, H k> / 64 = <q, k> */
      for (int g = 0; g < D / 64; ++g) {
        for (int j = 0; j < 64; ++j) {
          double acc = 0.0;
          for (int i = 0; i < 64; ++i) {
            int odd = __builtin_popcount((unsigned)(i & j)) & 1;
            acc += odd ? -qd[64 * g + i] : qd[64 * g + i];
          }
          row[64 * g + j] = acc / 8.0;
        }
      }
      for (int d = 0; d < D; ++d) qd[d] = row[d];
    }
    double m = -INFINITY;
    for (int j = 0; j <= last; ++j) {
      int block = block_table[(int64_t)b * max_blocks + j / 64];
      double acc = 0.0;
      for (int d = 0; d < D; ++d) acc += qd[d] * orc_dequant(p, 0, block, kvh, j % 64, d);
      z[j] = (double)softmax_scale * acc;
      if (z[j] > m) m = z[j];
    }
    double l = 0.0;
    for (int d = 0; d < D; ++d) row[d] = 0.0;
    for (int j = 0; j <= last; ++j) {
      int block = block_table[(int64_t)b * max_blocks + j / 64];
      double w = exp(z[j] - m);
      l += w;
      for (int d = 0; d < D; ++d) row[d] += w * orc_dequant(p, 1, block, kvh, j % 64, d);
    }
    double *o = out + (int64_t)i * D;
    for (int d = 0; d < D; ++d) o[d] = row[d] / l;
  }
  free(z);
  free(qd);
  free(row);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Array forms of the scalar conversions (for the pin tests)                 */
/* ------------------------------------------------------------------------ */

void orc_f32_to_f16_n(const float *x, uint16_t *y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_f32_to_f16_rne(x[i]);
}
void orc_f16_to_f32_n(const uint16_t *x, float *y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_f16_to_f32(x[i]);
}
void orc_bf16_to_f32_n(const uint16_t *x, float *y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_bf16_to_f32(x[i]);
}
void orc_f32_to_e4m3fn_n(const float *x, uint8_t *y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_f32_to_e4m3fn(x[i]);
}
void orc_e4m3fn_to_f32_n(const uint8_t *x, float *y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_e4m3fn_to_f32(x[i]);
}
/* rows of D values -> codes [n][D] and scales [n][D/64] (INT8, rk8v4 keys) or [n] (FP8) */
void orc_quant_rows(int fmt, const float *x, int64_t n, int D, uint8_t *codes, void *scales) {
  for (int64_t r = 0; r < n; ++r) {
    if (fmt == ORC_FMT_RK8V4)
      orc_quant_rk8v4_k(x + r * D, D, (int8_t *)codes + r * D, (uint16_t *)scales + r * (D / 64));
    else if (fmt == ORC_FMT_INT8_G64)
      orc_quant_int8_g64(x + r * D, D, (int8_t *)codes + r * D, (uint16_t *)scales + r * (D / 64));
    else
      orc_quant_fp8_row(x + r * D, D, codes + r * D, (float *)scales + r);
  }
}
void orc_h64_rotate_n(const float *x, float *y, int64_t ngroups) {
  for (int64_t g = 0; g < ngroups; ++g) orc_h64_rotate(x + 64 * g, y + 64 * g);
}
/* rk8v4 value rows: codes [n][D] (-7..7) and scales [n][D/32] */
void orc_quant_int4_rows(const float *x, int64_t n, int D, int8_t *codes, uint16_t *scales) {
  for (int64_t r = 0; r < n; ++r) orc_quant_int4_g32(x + r * D, D, codes + r * D, scales + r * (D / 32));
}
/* rk4v4 key rows: level indices [n][D] (0..15) and scales [n][D/64] */
void orc_quant_rk4v4_rows(const float *x, int64_t n, int D, uint8_t *idx, uint16_t *scales) {
  for (int64_t r = 0; r < n; ++r) orc_quant_rk4v4_k(x + r * D, D, idx + r * D, scales + r * (D / 64));
}
void orc_f32_to_bf16_n(const float *x, uint16_t *y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_f32_to_bf16_rne(x[i]);
}

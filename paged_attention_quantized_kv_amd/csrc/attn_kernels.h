// attn_kernels.h -- paged decode attention over the quantized page pool (device code).
//
// The result is out = softmax(q k^T * scale) v over the dequantized cache,
// which every decode step reads in full (NInfer-3090 README, "Choosing a KV
// format"); the context of each (sequence, KV head) is cut into
// chunks (split-K over the context) whose partial results are merged with
// log-sum-exp weights.
//
// Split kernel: a workgroup owns one chunk of one (sequence, KV head) and runs
// NTEAM teams of 4 waves; team t takes the chunk's pages t, t+NTEAM, ...  The
// 4 waves of a team share each page: wave w computes the scores of key tile w
// (16 keys) and accumulates the output for dim quarter w, so a wave holds a
// quarter of the page and a quarter of the output.  All T*G query rows of the
// KV head (T new tokens x G query heads of the group) ride along as the N
// dimension of 16x16x32 f16 matrix-core products, so every KV byte is read once:
//   S^T[key][row] = K[key][dim] * Q^T[dim][row]   (A = K codes, B = Q)
//   O^T[dim][row] = V^T[dim][key] * P^T[key][row] (A = V codes, B = softmax weights)
// Per page the team exchanges row maxima and softmax weights through LDS with one
// barrier (the weights are written optimistically against a lazily moved reference
// maximum; a rare second barrier settles a page whose maximum passed it); the next
// page's codes and scales are already in flight in a second register buffer.  K/V codes
// are converted to f16 exactly (int8 via byte permutes and one packed subtract, FP8 via
// the hardware converter, 4-bit codes via masks or a byte-permute table); softmax
// weights enter as f16 hi+lo pairs, fp32 queries as hi+lo, bf16 queries as one f16
// (exact in f16's normal range), so the rounding is fp32 summation.  The BF16 pool
// enters bf16 matrix-core products as it is.  The page layout (kvq.h) makes each
// 64-lane 16-byte load one contiguous KiB that lands in the operand registers.
//
// Prefill (T query rows per sequence, any T) runs either the split kernel's APP = 2
// instance (64-row blocks) or, for INT8 and FP8 pools with bf16 queries, prefill_kernel
// (128-row blocks whose waves own their rows; see there).
#pragma once

#include <type_traits>

#include "quant_row.h"

namespace kvq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));


__device__ inline f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// the BF16 format: bf16 operands, taken straight from the pool
__device__ inline f32x4 mfma16_bf(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// x = hi + mid + lo exactly enough for the BF16 format's P (24 significant bits): hi and
// mid are x and its residual cut to bf16 (exact residuals), lo the last residual rounded.
// Returns the bf16 pairs of two values x0, x1 packed per term.
__device__ inline void split_bf16x3(float x0, float x1, uint32_t &hi, uint32_t &mid, uint32_t &lo) {
  const float h0 = __uint_as_float(__float_as_uint(x0) & 0xFFFF0000u), h1 = __uint_as_float(__float_as_uint(x1) & 0xFFFF0000u);
  const float r0 = x0 - h0, r1 = x1 - h1;
  const float m0 = __uint_as_float(__float_as_uint(r0) & 0xFFFF0000u), m1 = __uint_as_float(__float_as_uint(r1) & 0xFFFF0000u);
  hi = __builtin_amdgcn_perm(__float_as_uint(h1), __float_as_uint(h0), 0x07060302u);
  mid = __builtin_amdgcn_perm(__float_as_uint(m1), __float_as_uint(m0), 0x07060302u);
  lo = f32_to_bf16_rne(r0 - m0) | (f32_to_bf16_rne(r1 - m1) << 16);
}

// Two signed int8 bytes of x (selected by `sel` after the sign flip) -> two
// exact f16 values.  Flipping the sign bit maps c to u = c + 128; the f16 with
// high byte 0x64 and low byte u is 1024 + u, so subtracting 1152 leaves c.
__device__ inline f16x2 i8pair(uint32_t xflip, uint32_t sel) {
  const uint32_t p = __builtin_amdgcn_perm(0x64646464u, xflip, sel);
  const f16x2 h = __builtin_bit_cast(f16x2, p);
  const _Float16 bias = static_cast<_Float16>(1152.0f);
  return h - f16x2{bias, bias};
}

// 8 code bytes (two dwords) -> 8 exact f16 values, in byte order.
template <int FMT>
__device__ inline f16x8 codes_to_f16(uint32_t w0, uint32_t w1) {
  if constexpr (FMT == 0) {
    const uint32_t x0 = w0 ^ 0x80808080u, x1 = w1 ^ 0x80808080u;
    const f16x2 a = i8pair(x0, 0x04010400u), b = i8pair(x0, 0x04030402u);
    const f16x2 c = i8pair(x1, 0x04010400u), d = i8pair(x1, 0x04030402u);
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  } else {
    // OCP E4M3FN -> f16 is exact (3 fraction bits, exponents 2^-9 .. 2^8)
    const f16x2 a = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false));
    const f16x2 b = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true));
    const f16x2 c = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false));
    const f16x2 d = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true));
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  }
}

// rk8v4 values: one 32-bit word holds the 4-bit codes (two's complement) of 8 keys,
// key q at bit 16*(q%2) + 4*(q/2), so masking with 0x000F000F after a shift of 4p
// gives keys 2p, 2p+1 in the two halves.  Flipping bit 3 of every nibble maps c to
// n = c + 8; the f16 with bits 0x6400 | n is 1024 + n, so subtracting 1032 leaves c.
__device__ inline f16x8 v4_to_f16(uint32_t w) {
  const uint32_t x = w ^ 0x88888888u;
  const _Float16 bias = static_cast<_Float16>(1032.0f);
  const f16x2 b2{bias, bias};
  const f16x2 a = __builtin_bit_cast(f16x2, (x & 0x000F000Fu) | 0x64006400u) - b2;
  const f16x2 b = __builtin_bit_cast(f16x2, ((x >> 4) & 0x000F000Fu) | 0x64006400u) - b2;
  const f16x2 c = __builtin_bit_cast(f16x2, ((x >> 8) & 0x000F000Fu) | 0x64006400u) - b2;
  const f16x2 d = __builtin_bit_cast(f16x2, ((x >> 12) & 0x000F000Fu) | 0x64006400u) - b2;
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// rk4v4 keys: one 32-bit word holds the 4-bit level indices of 8 dims of one key, byte b
// = dim b (low nibble) and dim b + 4 (high nibble).  Each index becomes its level's INT8
// code, biased by 128 (a 16-entry byte table read with two byte permutes and a per-byte
// select on bit 3), and the biased bytes become exact f16 as in i8pair.
__device__ inline uint32_t rk4_lut(uint32_t sel) {
  // biased codes c + 128 of the levels -127 -96 -75 -58 -44 -31 -18 -6 6 18 31 44 58 75 96 127
  constexpr uint32_t T0 = 0x46352001u, T1 = 0x7A6E6154u, T2 = 0xAC9F9286u, T3 = 0xFFE0CBBAu;
  const uint32_t s7 = sel & 0x07070707u;
  const uint32_t lo = __builtin_amdgcn_perm(T1, T0, s7), hi = __builtin_amdgcn_perm(T3, T2, s7);
  const uint32_t m = __builtin_amdgcn_perm(0u, 0u, ((sel >> 3) & 0x01010101u) | 0x0C0C0C0Cu);  // 0x00 / 0xFF
  return (hi & m) | (lo & ~m);
}
__device__ inline f16x8 k4_to_f16(uint32_t w) {
  const uint32_t a = rk4_lut(w & 0x0F0F0F0Fu), b = rk4_lut((w >> 4) & 0x0F0F0F0Fu);
  const f16x2 p0 = i8pair(a, 0x04010400u), p1 = i8pair(a, 0x04030402u);
  const f16x2 p2 = i8pair(b, 0x04010400u), p3 = i8pair(b, 0x04030402u);
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// x ~= hi + lo with hi = f16(x) rounded toward zero and lo = f16(x - hi): the
// pair carries ~21 significant bits.
__device__ inline void split_f16(float x0, float x1, f16x2 &hi, f16x2 &lo) {
  hi = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(x0, x1));
  lo = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(x0 - static_cast<float>(hi[0]),
                                                            x1 - static_cast<float>(hi[1])));
}

// The products p * s as an f16 hi+lo pair when p itself arrives as an f16 hi+lo pair
// (ph, pl) and s is fp16: hi = f16(ph*s); the residual ph*s - hi is exact in f16, and
// lo = f16(pl*s + residual).  Three packed f16 operations per pair of keys.
__device__ inline void scale_pair(f16x2 ph, f16x2 pl, f16x2 s, f16x2 &hi, f16x2 &lo) {
  hi = ph * s;
  const f16x2 r = __builtin_elementwise_fma(ph, s, -hi);
  lo = __builtin_elementwise_fma(pl, s, r);
}

// The same split of the products p * s (s in fp16): hi = f16(p*s) toward zero, lo =
// f16(p*s - hi) with the residual taken from the unrounded product; each product and
// residual is one mixed-precision fma.
__device__ inline void split_scaled(float p0, float p1, f16x2 s, f16x2 &hi, f16x2 &lo) {
  const float s0 = static_cast<float>(s[0]), s1 = static_cast<float>(s[1]);
  hi = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(__builtin_fmaf(p0, s0, 0.0f), __builtin_fmaf(p1, s1, 0.0f)));
  lo = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(__builtin_fmaf(p0, s0, -static_cast<float>(hi[0])),
                                                            __builtin_fmaf(p1, s1, -static_cast<float>(hi[1]))));
}

// Element i of the query tensor, widened to fp32 (bf16 widening is exact).
template <bool BF16>
__device__ inline float load_q(const void *q, size_t i) {
  if constexpr (BF16) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(q)[i]) << 16);
  return static_cast<const float *>(q)[i];
}

__device__ inline f16x8 lds_f16x8(const uint4 *p) { return __builtin_bit_cast(f16x8, *p); }

// Butterfly steps across the 16-lane rows of a wave without LDS: lane l gets
// op(x[l], x[l ^ 16]) and op(x[l], x[l ^ 32]) via the gfx950 row/half swaps.
__device__ inline float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 2^x with the hardware exponential: exact at 0 and -inf; results below the
// normal range (weights under 2^-126 of the running maximum) may flush to zero.
__device__ inline float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Rescaling threshold of the online softmax, log2 units (see the softmax phase).
constexpr float kLazy = 8.0f;

// ---- Exponent offsets of the P·V operands.
//
// The weight of key j enters the matrix cores as the f16 pair of p_j * s_j (p_j its softmax
// weight against the running reference, s_j its V scale), and f16 has only ~40 binades,
// 2^-24 .. 2^16.  Both factors span far more: weights reach down to where thousands of
// near-uniform keys under a dominant one (an attention sink) still sum to a visible share
// of the output, and scales are whatever the data make them.  Two powers of two keep the
// products in the normal range without any per-key work:
//   - kWeightExp: the weights are formed as exp2(z - m + kWeightExp), so with the lazy
//     reference (weights <= 2^kLazy) they stay <= 2^15 and their f16 hi + lo pair carries
//     21 bits down to p ~ 2^-11 and stays exact to 2^-31 absolute below; the row sums carry
//     the same offset, so the normalized output does not see it.
//   - the V-scale exponent E (per wave, only ever lowered within a chunk): the scales the
//     products use are s * 2^E, with E set from the largest scale the wave has seen so
//     that the largest product stays below 2^15; the accumulators carry 2^E, taken out
//     when the chunk's output is written.  When a page brings a larger scale, E drops and
//     the accumulators are rescaled (rare: once per chunk on typical data).
// The FP8 pool keeps its weights in fp32 up to the product, so there both offsets fold into
// the exponent of the weights and the row sums (E chosen so that p * s stays below 2^15).
constexpr int kWeightExp = 15 - static_cast<int>(kLazy);  // 7
constexpr int kVexpMax = 14, kVexpMin = -16;               // E range of fp16 scales (2^E is an f16)
constexpr int kFp8ExpMax = 30, kFp8ExpMin = -60;           // E range of fp32 scales

// The largest of the finite non-negative fp16 scales packed in N words of this lane, as fp16
// bits in the low half (the high half zero): a three-input tree over the words (IEEE
// maximum: the scales are finite, the poison of unwritten slots is zeroed before), then
// the two halves.
template <int N>
__device__ inline uint32_t lane_max_f16_scales(const uint32_t (&w)[N]) {
  f16x2 t[N];
#pragma unroll
  for (int i = 0; i < N; ++i) t[i] = __builtin_bit_cast(f16x2, w[i]);
  int n = N;
#pragma unroll
  for (int round = 0; round < 4; ++round) {
    if (n > 1) {
      int k = 0;
#pragma unroll
      for (int i = 0; i < N; i += 3) {
        if (i < n) {
          f16x2 x = t[i];
          if (i + 1 < n) x = __builtin_elementwise_maximum(x, t[i + 1]);
          if (i + 2 < n) x = __builtin_elementwise_maximum(x, t[i + 2]);
          t[k++] = x;
        }
      }
      n = k;
    }
  }
  const f16x2 x = __builtin_elementwise_maximum(t[0], f16x2{t[0][1], t[0][0]});
  return __builtin_bit_cast(uint32_t, x) & 0xFFFFu;
}

// The same for non-negative fp32 scales: this lane's largest as fp32 bits.
template <int N>
__device__ inline uint32_t lane_max_f32_scales(const uint32_t (&w)[N]) {
  uint32_t t[N];
#pragma unroll
  for (int i = 0; i < N; ++i) t[i] = w[i];
#pragma unroll
  for (int h = 1; h < N; h <<= 1)
#pragma unroll
    for (int i = 0; i + h < N; i += 2 * h) t[i] = max(t[i], t[i + h]);
  return t[0];
}

// The largest u of the wave, in every lane: across the four 16-lane groups with lane swaps,
// as 32-bit integers (non-negative IEEE values order like their bit patterns; hipcc 7.2
// drops a packed 16-bit max of the two results of a lane swap, a 32-bit max it keeps).
__device__ inline uint32_t wave_max_u32(uint32_t u) {
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  u = max(r[0], r[1]);
  r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return max(r[0], r[1]);
}

// E for the largest scale (wave-uniform result): fp16 scales (bits h) get smax * 2^E in
// [1/2, 1), so products with weights <= 2^15 stay below 2^15; fp32 (FP8) scales get
// smax * 2^E in [2^6, 2^7), for weights <= 2^kLazy.  Zero or subnormal maxima take the top
// of the range.  Clamped to the ranges above.
__device__ inline int scale_exponent_f16(uint32_t hbits) {
  const int ef = static_cast<int>(__builtin_amdgcn_readfirstlane(hbits) >> 10) & 0x1F;  // f16 exponent field
  return max(min(14 - ef, kVexpMax), kVexpMin);
}
__device__ inline int scale_exponent_f32(uint32_t fbits) {
  const int e = static_cast<int>(__builtin_amdgcn_readfirstlane(fbits) >> 23) & 0xFF;  // fp32 exponent field
  return max(min(133 - e, kFp8ExpMax), kFp8ExpMin);
}
// The smallest scale bits whose exponent asks for an E below cur: for fp16 scales
// E < cur <=> 14 - ef < cur <=> bits >= (15 - cur) << 10; for fp32 scales E < cur <=>
// 133 - e < cur <=> bits >= (134 - cur) << 23 (no bits do at the bottom of the range).
__device__ inline uint32_t lower_threshold_f16(int cur) {
  return cur <= kVexpMin ? 0xFFFFFFFFu : static_cast<uint32_t>(15 - cur) << 10;
}
__device__ inline uint32_t lower_threshold_f32(int cur) {
  return cur <= kFp8ExpMin ? 0xFFFFFFFFu : static_cast<uint32_t>(134 - cur) << 23;
}

// Query rows enter the matrix cores as f16, whose range (2^-24 .. 65504) is far narrower than
// bf16's or fp32's.  Each row is scaled by 2^-s before the conversion, s chosen from its
// largest |element| (fp32 bits mbits) so that the largest lands in [2^14, 2^15); the row's
// scores take 2^s back.  A bf16 row whose elements all lie within 2^28 of its largest thus
// enters exactly (and an fp32 row as its hi + lo pair); smaller elements, whose products
// are below 2^-28 of the largest one's, keep 2^-24 of it absolute.  An all-zero row takes s = 0.
__device__ inline int q_row_exp(uint32_t mbits) {
  if (mbits == 0) return 0;
  return max(min(static_cast<int>((mbits >> 23) & 0xFFu) - 127 - 14, 100), -100);
}

// 2^E as two packed f16 (E in [kVexpMin, kVexpMax]; 2^-15 and 2^-16 are subnormal).
__device__ inline uint32_t f16x2_pow2(int E) {
  const uint32_t h = (E >= -14) ? static_cast<uint32_t>(E + 15) << 10 : (0x400u >> (-14 - E));
  return h | (h << 16);
}

// One wave's share of one page: its K tile (16 keys x all dims) and its V dim
// tiles (all 64 keys), with their scales.  rk8v4 (FMT 2): K as INT8; V as 4-bit codes,
// one 16-byte load per pair of dim tiles, and the fp16 scales of two 32-dim groups.
template <int D, int FMT>
struct PageRegs {
  static constexpr int G64 = D / 64, DPW = D / 64;  // dim tiles per wave = D/16/4
  // BF16 (FMT 4): 32 bytes of K per (key, 16 dims) and of V per (dim, 16 keys), no scales
  static constexpr int KSN = (FMT == 1 || FMT == 4) ? 1 : (D / 128);
  static constexpr int KN = (FMT == 3) ? G64 / 2 : (FMT == 4 ? 2 * G64 : G64);  // rk4v4: 16 bytes per pair of 64-dim groups
  static constexpr int VN = (FMT == 2 || FMT == 3) ? DPW / 2 : (FMT == 4 ? 2 * DPW : DPW);
  static constexpr int VSN = (FMT == 0) ? 2 : (FMT == 1 ? 4 : (FMT == 4 ? 1 : DPW));
  uint4 k[KN];
  uint4 v[VN];
  uint4 ks[KSN];
  uint4 vs[VSN];
};

// The pages are streamed once per call: load them with the non-temporal hint.
__device__ inline uint4 ld_stream(const uint4 *p) {
#if KVQ_NT_LOADS
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
#else
  return *p;
#endif
}

// The K half of one wave's share of a page (its key tile and the tile's scales) and
// the V half (its dim tiles and all 64 keys' scales), issued separately so the loads of
// the next page spread over the current one.
template <int D, int FMT>
__device__ inline void load_k_part(PageRegs<D, FMT> &r, const AttnArgs &a, int pg_any, int wave, int lane, int q4) {
  constexpr int G64 = D / 64, NCH = D / 16;
  const size_t pg = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(pg_any));  // wave-uniform page
  const uint4 *kp = reinterpret_cast<const uint4 *>(a.k_codes + pg * kPage * D);
  if constexpr (FMT == 4) {  // bf16 keys: the INT8 unit u of this lane holds 16 dims, here 2 x 16 bytes
    const uint4 *kp16 = reinterpret_cast<const uint4 *>(a.k_codes + pg * kPage * D * 2);
#pragma unroll
    for (int cg = 0; cg < G64; ++cg) {
      const int u = (wave * NCH + 4 * cg) * 16 + lane;
      r.k[2 * cg] = ld_stream(kp16 + 2 * u);
      r.k[2 * cg + 1] = ld_stream(kp16 + 2 * u + 1);
    }
    return;
  } else if constexpr (FMT == 3) {  // 4-bit keys: (key tile, group pair) units of 1 KiB, 16 bytes per lane
    const uint4 *kp4 = reinterpret_cast<const uint4 *>(a.k_codes + pg * kPage * (D / 2));
#pragma unroll
    for (int p = 0; p < G64 / 2; ++p) r.k[p] = ld_stream(kp4 + (wave * (G64 / 2) + p) * 64 + lane);
  } else {
#pragma unroll
    for (int cg = 0; cg < G64; ++cg) r.k[cg] = ld_stream(kp + (wave * NCH + 4 * cg) * 16 + lane);
  }
  if constexpr (FMT != 1) {
    const uint4 *ksp = reinterpret_cast<const uint4 *>(static_cast<const _Float16 *>(a.k_scales) + pg * D);
#pragma unroll
    for (int j = 0; j < PageRegs<D, FMT>::KSN; ++j) r.ks[j] = ksp[(q4 * 4 + wave) * PageRegs<D, FMT>::KSN + j];
  } else {
    const uint4 *ksp = reinterpret_cast<const uint4 *>(static_cast<const float *>(a.k_scales) + pg * kPage);
    r.ks[0] = ksp[q4 * 4 + wave];
  }
}

template <int D, int FMT>
__device__ inline void load_v_part(PageRegs<D, FMT> &r, const AttnArgs &a, int pg_any, int wave, int lane, int q4) {
  constexpr int G64 = D / 64, DPW = D / 64;
  const size_t pg = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(pg_any));
  if constexpr (FMT == 4) {  // bf16 values: the INT8 unit u of this lane (16 keys of one dim), here 2 x 16 bytes
    const uint4 *vp16 = reinterpret_cast<const uint4 *>(a.v_codes + pg * kPage * D * 2);
#pragma unroll
    for (int j = 0; j < DPW; ++j) {
      const int u = (wave * DPW + j) * 64 + lane;
      r.v[2 * j] = ld_stream(vp16 + 2 * u);
      r.v[2 * j + 1] = ld_stream(vp16 + 2 * u + 1);
    }
    return;
  }
  if constexpr (FMT == 2 || FMT == 3) {  // 4-bit codes: tile pair p of the wave is one KiB, 16 bytes per lane
    const uint4 *vp = reinterpret_cast<const uint4 *>(a.v_codes + pg * kPage * (D / 2));
#pragma unroll
    for (int p = 0; p < DPW / 2; ++p) r.v[p] = ld_stream(vp + (wave * (DPW / 2) + p) * 64 + lane);
    const uint4 *vsp = reinterpret_cast<const uint4 *>(static_cast<const _Float16 *>(a.v_scales) + pg * (kPage * D / 32));
#pragma unroll
    for (int p = 0; p < DPW / 2; ++p)
#pragma unroll
      for (int j = 0; j < 2; ++j) r.vs[2 * p + j] = vsp[(q4 * (D / 32) + wave * (DPW / 2) + p) * 2 + j];
    return;
  }
  const uint4 *vp = reinterpret_cast<const uint4 *>(a.v_codes + pg * kPage * D);
#pragma unroll
  for (int j = 0; j < DPW; ++j) r.v[j] = ld_stream(vp + (wave * DPW + j) * 64 + lane);
  if constexpr (FMT == 0) {
    const uint4 *vsp = reinterpret_cast<const uint4 *>(static_cast<const _Float16 *>(a.v_scales) + pg * D);
    const int g = (wave * DPW) / 4;  // the 64-dim group of this wave's dims
#pragma unroll
    for (int j = 0; j < 2; ++j) r.vs[j] = vsp[(q4 * G64 + g) * 2 + j];
  } else {
    const uint4 *vsp = reinterpret_cast<const uint4 *>(static_cast<const float *>(a.v_scales) + pg * kPage);
#pragma unroll
    for (int j = 0; j < 4; ++j) r.vs[j] = vsp[q4 * 4 + j];
  }
}

template <int D, int FMT>
__device__ inline void load_page(PageRegs<D, FMT> &r, const AttnArgs &a, int pg_any, int wave, int lane, int q4) {
  load_k_part<D, FMT>(r, a, pg_any, wave, lane, q4);
  load_v_part<D, FMT>(r, a, pg_any, wave, lane, q4);
}

__device__ inline void f16x2_to_f32(uint32_t w, float &x, float &y) {
  const f16x2 h = __builtin_bit_cast(f16x2, w);
  x = static_cast<float>(h[0]);
  y = static_cast<float>(h[1]);
}

// Balanced chunking of a call of 2..kMaxBalancedSeqs sequences.  Every (sequence, KV head)
// is cut into chunks of one common length of pp pages (an even count, whole rounds of the
// teams), the smallest for which the call's chunks, sum over (b, kvh) of ceil(pages_b / pp),
// number at most kTargetWgs (one workgroup per compute unit, so they all run at once), and at
// most kMaxChunkPages.  A sequence so gets chunks in proportion to its own length.  Chunk c of
// unit (b, kvh) is split workgroup and partial slot first_b + kvh * n_b + c, first_b =
// Hkv * (n_0 + .. + n_{b-1}).  A sequence whose length is out of range counts as one chunk of
// no pages (its rows come out NaN).  Lane b of the wave gets sequence b's first_b and n_b;
// every lane the common chunk length and the slot count.
struct BalancedChunks {
  int tps, first, n, total;
};
__device__ inline int wave_sum(int x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ inline BalancedChunks balanced_chunks(const AttnArgs &a, int lane) {
  int pages = 0;
  if (lane < a.num_seqs) {
    const int L = a.seq_lens[lane];
    if (L >= a.T && L <= a.max_seq_len && L <= static_cast<long>(a.max_blocks) * kPage) pages = (L + kPage - 1) / kPage;
  }
  auto even = [](int x) { return x + (x & 1); };
  auto count = [&](int q) {  // the call's chunks at q pages per chunk
    return wave_sum(lane < a.num_seqs ? max(1, (pages + q - 1) / q) : 0) * a.num_kv_heads;
  };
  const long P = static_cast<long>(wave_sum(pages)) * a.num_kv_heads;
  int pp = max(even(static_cast<int>((P + kTargetWgs - 1) / kTargetWgs)), kTeams);
  if (count(pp) > kTargetWgs) {  // rounding up per unit added chunks: search the smallest length that fits
    int hi = pages;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) hi = max(hi, __shfl_xor(hi, o));
    hi = max(even(hi), pp);  // one chunk per unit: the fewest chunks there can be
    int lo = pp;             // count(lo) > kTargetWgs
    while (hi - lo > 2) {
      const int mid = even((lo + hi) / 2);
      if (mid >= hi) break;
      if (count(mid) <= kTargetWgs) hi = mid; else lo = mid;
    }
    pp = hi;
  }
  pp = min(pp, kMaxChunkPages);
  const int n = (lane < a.num_seqs) ? max(1, (pages + pp - 1) / pp) : 0;
  int incl = n * a.num_kv_heads;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  BalancedChunks c;
  c.tps = pp * kPage;
  c.first = incl - n * a.num_kv_heads;
  c.n = n;
  c.total = __shfl(incl, 63);
  return c;
}

template <int D, int NT, int NTEAM, int QP>
struct Smem {
  static constexpr int ROWS = 16 * NT, PST = 64 + 4, G64 = D / 64;
  static constexpr int QS = NT * G64 * 2 * QP * 64;            // Q operand entries (uint4)
  static constexpr int PB = NTEAM * 2 * ROWS * PST;             // softmax-weight exchange (floats)
  static constexpr int FIN = (NTEAM > 1 ? NTEAM - 1 : 1) * ROWS * (D + 4);  // team merge (floats), aliases pb
  static constexpr int PBF = PB > FIN ? PB : FIN;
};

// APP: 1 = also quantize and append the T new rows of each sequence (the fused
// decode step; the source dtype is the query dtype), 0 = the cache is complete,
// 2 = prefill: the query rows come in blocks of 16*NT rows (grid y = row block * Hkv
// + KV head), chunks hold up to kMaxPrefillChunkPages pages, and with one chunk per
// row block the normalized rows go straight to out.
// QLO: 0 = bf16 queries entering as one f16 each; 1 = fp32 queries as f16 hi + lo;
// 2 = bf16 queries rotated for rk8v4 keys (FMT 2), which no longer fit one f16: hi + lo.
template <int D, int NT, int FMT, int QLO, int NTEAM, int APP>
__global__ __launch_bounds__(256 * NTEAM, 1) void attn_split_kernel(AttnArgs a) {
  constexpr int G64 = D / 64, NCH = D / 16, DPW = D / 64;
  constexpr int QP = QLO ? 2 : 1;
  constexpr int KF = (FMT == 2) ? 0 : FMT;  // key code format: rk8v4 keys are INT8 group-64
  static_assert(FMT != 2 && FMT != 3 || QLO != 0, "rotated queries need the lo part");
  using SM = Smem<D, NT, NTEAM, QP>;
  constexpr int ROWS = SM::ROWS, PST = SM::PST;
  __shared__ uint4 qs[SM::QS];
  __shared__ float4 pbuf4[SM::PBF / 4];
  __shared__ float4 lds_mx[NTEAM][2][ROWS];  // per row: the 4 waves' page maxima
  __shared__ int32_t lds_over[2][4 * NTEAM];  // per wave: a page maximum passed the reference by > kLazy
  __shared__ float lds_l[NTEAM][4][ROWS];
  __shared__ float lds_m[NTEAM][ROWS];
  constexpr int MAXPG = (APP == 2) ? kMaxPrefillChunkPages : kMaxChunkPages;
  __shared__ int32_t lds_pg[MAXPG];  // pool page (block * Hkv + kvh) of each page of the chunk
  __shared__ uint32_t lds_qmax[ROWS];  // per query row: the largest |element| (fp32 bits)
  float *pbuf = reinterpret_cast<float *>(pbuf4);

  const int tid = threadIdx.x, lane = tid & 63, wave = (tid >> 6) & 3, team = tid >> 8;
  const int q4 = lane >> 4, c16 = lane & 15;
  int split = blockIdx.x, kvh = blockIdx.y % a.num_kv_heads, b = blockIdx.z;
  // first query row (t*G + g) of this block; prefill row blocks go out last first, since the
  // later rows see the most keys (longest workgroups first keeps the last round short)
  const int row0 = (a.row_blocks - 1 - static_cast<int>(blockIdx.y) / a.num_kv_heads) * ROWS;
  int tps = a.tokens_per_split;
  size_t part = (static_cast<size_t>(b) * a.num_kv_heads + kvh) * a.n_splits + split;  // partial slot
  bool direct = a.direct_out != 0;  // normalized rows to out, no partials
  if constexpr (APP != 2) {
    if (a.balanced != 0) {  // this workgroup's (sequence, KV head, chunk) from the actual lengths
      const BalancedChunks c = balanced_chunks(a, lane);
      const int w = blockIdx.x;
      const unsigned long long m = __ballot(lane < a.num_seqs && c.first <= w && w < c.first + c.n * a.num_kv_heads);
      if (m == 0) return;  // past the call's chunks
      b = __ffsll(static_cast<long long>(m)) - 1;
      const int first = __shfl(c.first, b), nb = __shfl(c.n, b);
      kvh = (w - first) / nb;
      split = (w - first) % nb;
      tps = c.tps;
      part = w;
      direct = a.direct_single != 0 && nb == 1;  // a one-chunk sequence: the merge skips it
    }
  }
  const int L = a.seq_lens[b];
  if (L < a.T || L > a.max_seq_len || L > static_cast<long>(a.max_blocks) * kPage) {  // the merge writes NaN rows
    if (a.direct_out != 0 && split == 0) {  // no merge: write them here
      for (int e = threadIdx.x; e < ROWS * D; e += blockDim.x) {
        const int r = row0 + e / D;
        if (r < a.rows)
          a.out[((static_cast<size_t>(b) * a.T + r / a.group) * a.num_q_heads + kvh * a.group + r % a.group) * D +
                e % D] = NAN;
      }
    }
    return;
  }
  const int R = a.rows;  // query rows of the KV head; this block holds rows row0 .. row0 + ROWS - 1
  // keys this block's rows can see: row r = t*G + g sees positions 0 .. L - T + t
  const int lim = (APP == 2) ? L - a.T + (min(row0 + ROWS, R) - 1) / a.group + 1 : L;
  const int lo_last = L - a.T + row0 / a.group;  // the last key the block's first row sees
  const int tok0 = split * tps;
  if (tok0 >= lim) return;  // chunk past every key of these rows: the merge skips it
  const int tok1 = min(tok0 + tps, lim);
  const int page0 = tok0 / kPage, page1 = (tok1 + kPage - 1) / kPage;

  // ---- the chunk's block ids -> pool pages in LDS (an invalid id reads block 0 and flags the chunk)
  bool bad = false;
  const int32_t *bt = a.block_table + static_cast<size_t>(b) * a.max_blocks;
  for (int i = tid; i < page1 - page0; i += 256 * NTEAM) {
    const int blk = bt[page0 + i];
    const bool ok = (blk >= 0) && (blk < a.num_blocks);
    bad |= !ok;
    lds_pg[i] = (ok ? blk : 0) * a.num_kv_heads + kvh;
  }
  if (tid < ROWS) lds_qmax[tid] = 0u;
  bad = __syncthreads_or(bad ? 1 : 0) != 0;

  const int n_it = (page1 - page0 + NTEAM - 1) / NTEAM;
  // pool page of iteration it for this team (clamped: iterations past the team's last
  // page reload that page and skip the math)
  auto page_of = [&](int it) -> int { return lds_pg[min(it * NTEAM + team, page1 - page0 - 1)]; };
  PageRegs<D, FMT> rA, rB;

  // ---- fused decode step: the new rows at positions L-T .. L-1 that fall in this chunk
  // (K and V of each, one wave per row).  When their first page is not loaded before
  // iteration 3, the source rows are read now, quantized and stored during page 0, and
  // the writing waves wait for their stores at the end of page 0, before the barrier
  // that precedes every load of iteration 3 on; otherwise they are written here.
  constexpr int NW = 4 * NTEAM, RPW = (16 + NW - 1) / NW;  // T <= 8: at most 16 rows
  [[maybe_unused]] AppendArgs aa;
  [[maybe_unused]] float xr[RPW][G64];
  [[maybe_unused]] int blk_r[RPW];
  int t_lo = 0, n_rows = 0;
  bool defer = false;
  if constexpr (APP == 1) {
    aa.k_new = a.k_new;
    aa.v_new = a.v_new;
    aa.k_codes = const_cast<uint8_t *>(a.k_codes);
    aa.v_codes = const_cast<uint8_t *>(a.v_codes);
    aa.k_scales = const_cast<void *>(a.k_scales);
    aa.v_scales = const_cast<void *>(a.v_scales);
    aa.block_table = a.block_table;
    aa.start_pos = nullptr;
    aa.start_back = 0;
    aa.max_len = 0;
    aa.num_seqs = a.num_seqs;
    aa.n_new = a.T;
    aa.num_kv_heads = a.num_kv_heads;
    aa.max_blocks = a.max_blocks;
    aa.num_blocks = a.num_blocks;
    t_lo = max(0, tok0 - (L - a.T));
    n_rows = 2 * max(0, min(a.T, tok1 - (L - a.T)) - t_lo);
    defer = (max((L - a.T) / kPage, page0) - page0) / NTEAM >= 3;
    if (defer) {
#pragma unroll
      for (int k = 0; k < RPW; ++k) {
        const int r = (tid >> 6) + k * NW;
        blk_r[k] = -1;
        if (r < n_rows) {
          const int t = t_lo + (r >> 1);
          blk_r[k] = bt[(L - a.T + t) / kPage];
          load_row<D, QLO == 1 ? 0 : 1>(aa, b, t, kvh, r & 1, lane, xr[k]);
        }
      }
    }
  }
  // the first pages load while the queries are staged (and, for the fused step, the new
  // rows read) -- unless one of them holds new rows, which must be written first
  const bool early = (APP != 1) || (page0 + NTEAM - 1 < (L - a.T) / kPage);
  if (early && n_it > 0) load_k_part<D, FMT>(rA, a, page_of(0), wave, lane, q4);

  // ---- queries -> LDS in B-operand order: entry (nt, cg, hk, hl, lane) holds dims
  // 64cg + 16(lane/16) + 8hk + 0..7 of row 16nt + lane%16, as f16 hi (hl=0) or lo (hl=1).
  // Two passes: the largest |element| of every row (LDS max), then the rows scaled by
  // 2^-q_row_exp into f16 (the BF16 pool takes bf16 operands and needs no scaling).
  if constexpr (FMT == 2 || FMT == 3) {
    // rk8v4, rk4v4: the keys are stored rotated by H64/8 per 64-dim group, so each 64-dim group
    // of a query row is rotated by the same matrix (butterflies in fp32, one thread per
    // (row, group)) before it is split into f16 hi + lo
    static_assert(ROWS * G64 <= 256 * NTEAM, "one rotation task per thread");
    const int rl = tid / G64, cg = tid % G64, r = row0 + rl;
    const bool live = tid < ROWS * G64;
    float v[64];
    if (live && r < R) {
      const int t = r / a.group, hq = kvh * a.group + r % a.group;
      const size_t qb = ((static_cast<size_t>(b) * a.T + t) * a.num_q_heads + hq) * D + 64 * cg;
#pragma unroll
      for (int i = 0; i < 64; ++i) v[i] = load_q<QLO != 1>(a.q, qb + i);
    } else {
#pragma unroll
      for (int i = 0; i < 64; ++i) v[i] = 0.0f;
    }
#pragma unroll
    for (int hh = 1; hh < 64; hh <<= 1)
#pragma unroll
      for (int i = 0; i < 64; ++i)
        if ((i & hh) == 0) {
          const float u = v[i], w = v[i + hh];
          v[i] = u + w;
          v[i + hh] = u - w;
        }
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < 64; ++i) mx = max(mx, __float_as_uint(v[i]) & 0x7FFFFFFFu);
    if (live) atomicMax(&lds_qmax[rl], mx);
    __syncthreads();
    if (live) {
      // the rotation's 1/8 and the row's 2^-s in one power of two
      const float f = __builtin_ldexpf(0.125f, -q_row_exp(__float_as_uint(__uint_as_float(lds_qmax[rl]) * 0.125f)));
#pragma unroll
      for (int jh = 0; jh < 8; ++jh) {  // dims 8jh .. 8jh+7 of the group: lane 16(jh/2) + rl%16, hk = jh%2
        f16x2 hi[4], lo[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) split_f16(v[8 * jh + 2 * j] * f, v[8 * jh + 2 * j + 1] * f, hi[j], lo[j]);
        const int idx = (((rl / 16) * G64 + cg) * 2 + (jh & 1)) * QP * 64 + 16 * (jh >> 1) + (rl % 16);
        qs[idx] = __builtin_bit_cast(uint4, f16x8{hi[0][0], hi[0][1], hi[1][0], hi[1][1], hi[2][0], hi[2][1], hi[3][0], hi[3][1]});
        qs[idx + 64] = __builtin_bit_cast(uint4, f16x8{lo[0][0], lo[0][1], lo[1][0], lo[1][1], lo[2][0], lo[2][1], lo[3][0], lo[3][1]});
      }
    }
  } else {
    constexpr int QN = NT * G64 * 2 * 64, QIT = (QN + 256 * NTEAM - 1) / (256 * NTEAM);
    float xq[QIT][8];
#pragma unroll
    for (int k = 0; k < QIT; ++k) {
      const int e = tid + k * 256 * NTEAM;
      const int ln = e & 63, hk = (e >> 6) & 1, cg = (e >> 7) % G64, nt = (e >> 7) / G64;
      const int r = row0 + 16 * nt + (ln & 15);
      const int d0 = 64 * cg + 16 * (ln >> 4) + 8 * hk;
      uint32_t mx = 0;
      if (e < QN && r < R) {
        const int t = r / a.group, hq = kvh * a.group + r % a.group;
        const size_t qb = ((static_cast<size_t>(b) * a.T + t) * a.num_q_heads + hq) * D + d0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xq[k][j] = load_q<QLO != 1>(a.q, qb + j);
          mx = max(mx, __float_as_uint(xq[k][j]) & 0x7FFFFFFFu);
        }
        if constexpr (FMT != 4) atomicMax(&lds_qmax[16 * nt + (ln & 15)], mx);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) xq[k][j] = 0.0f;
      }
    }
    if constexpr (FMT != 4) __syncthreads();
#pragma unroll
    for (int k = 0; k < QIT; ++k) {
      const int e = tid + k * 256 * NTEAM;
      if (e >= QN) continue;
      const int ln = e & 63, hk = (e >> 6) & 1, cg = (e >> 7) % G64, nt = (e >> 7) / G64;
      const float f = (FMT == 4) ? 1.0f : __builtin_ldexpf(1.0f, -q_row_exp(lds_qmax[16 * nt + (ln & 15)]));
      f16x2 hi[4], lo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // QLO = 1 for fp32 queries (hi + lo), 0 for bf16 queries (one f16, exact once scaled)
        const float x0 = xq[k][2 * j] * f, x1 = xq[k][2 * j + 1] * f;
        if constexpr (FMT == 4) {
          // BF16 pool: bf16 operands; a bf16 query is exact, an fp32 one is bf16 hi (cut)
          // + lo (the exact residual rounded)
          const uint32_t h0 = __float_as_uint(x0) & 0xFFFF0000u, h1 = __float_as_uint(x1) & 0xFFFF0000u;
          const uint32_t l = f32_to_bf16_rne(x0 - __uint_as_float(h0)) | (f32_to_bf16_rne(x1 - __uint_as_float(h1)) << 16);
          hi[j] = __builtin_bit_cast(f16x2, (h0 >> 16) | h1);
          lo[j] = __builtin_bit_cast(f16x2, QLO ? l : 0u);
        } else if constexpr (QLO) {
          split_f16(x0, x1, hi[j], lo[j]);
        } else {
          hi[j] = f16x2{static_cast<_Float16>(x0), static_cast<_Float16>(x1)};
          lo[j] = f16x2{0, 0};
        }
      }
      const int idx = ((nt * G64 + cg) * 2 + hk) * QP * 64 + ln;
      qs[idx] = __builtin_bit_cast(uint4, f16x8{hi[0][0], hi[0][1], hi[1][0], hi[1][1], hi[2][0], hi[2][1], hi[3][0], hi[3][1]});
      if constexpr (QLO)
        qs[idx + 64] = __builtin_bit_cast(uint4, f16x8{lo[0][0], lo[0][1], lo[1][0], lo[1][1], lo[2][0], lo[2][1], lo[3][0], lo[3][1]});
    }
  }
  if constexpr (APP == 1) {
    if (!defer) {
      for (int r = (tid >> 6); r < n_rows; r += NW) {
        const int t = t_lo + (r >> 1);
        const long pos = static_cast<long>(L) - a.T + t;
        const int blk = bt[pos / kPage];
        if (blk >= 0 && blk < a.num_blocks) quant_row<FMT, D, QLO == 1 ? 0 : 1>(aa, b, t, kvh, r & 1, pos, blk, lane);
      }
      // a wave that wrote rows waits until its stores have reached L2, so every wave of this
      // workgroup loads the new rows after the barrier below (no other workgroup reads them)
      if ((tid >> 6) < n_rows) __builtin_amdgcn_s_waitcnt(0);
    }
  }
  // the first page's V half goes out after the staging, so its K half arrives first
  if (early && n_it > 0) load_v_part<D, FMT>(rA, a, page_of(0), wave, lane, q4);
  __syncthreads();
  if (!early && n_it > 0) load_page<D, FMT>(rA, a, page_of(0), wave, lane, q4);

  // ---- per-lane state; this lane's query row is 16nt + c16
  float m[NT], lsum[NT], qsc[NT];
  int last[NT];
  f32x4 o[NT][DPW];
  // exponent offsets of the P·V operands (see kWeightExp): fp16-scale formats carry kWeightExp
  // in the weights and row sums and the wave's V-scale exponent vexp in o; FP8 carries vexp
  // in the weights, row sums and o alike; BF16 needs neither (its weights stay fp32-ranged)
  constexpr bool F16PAIR = (FMT == 0 || FMT == 2 || FMT == 3);
  int vexp = (FMT == 1) ? kFp8ExpMax : kVexpMax;  // wave-uniform
  auto wexp = [&]() -> float { return F16PAIR ? static_cast<float>(kWeightExp) : (FMT == 1 ? static_cast<float>(vexp) : 0.0f); };
  // wave-uniform companions of vexp, recomputed only when it moves: the scale bits from
  // which a page asks for a lower exponent, and 2^vexp as two packed f16
  uint32_t vth = (FMT == 1) ? lower_threshold_f32(vexp) : lower_threshold_f16(vexp);
  uint32_t e2bits = f16x2_pow2(F16PAIR ? vexp : 0);
  // V scales of slots at or past L (never written: poison) -> 0, on pages that hold such slots;
  // the V-scale words of a lane group hold keys 16(2j + e/4) + 4 q4 + e%4 (e: the element of
  // word j, 8 fp16 or 4 fp32 per uint4) for every format with scales
  auto zero_unwritten_scales = [&](PageRegs<D, FMT> &pr, int p) {
    const int kbase = p * kPage + 4 * q4;
    if constexpr (FMT == 1) {  // vs[j]: keys 16 j + 4 q4 + i
#pragma unroll
      for (int j = 0; j < PageRegs<D, FMT>::VSN; ++j) {
        pr.vs[j].x = (kbase + 16 * j + 0 < L) ? pr.vs[j].x : 0u;
        pr.vs[j].y = (kbase + 16 * j + 1 < L) ? pr.vs[j].y : 0u;
        pr.vs[j].z = (kbase + 16 * j + 2 < L) ? pr.vs[j].z : 0u;
        pr.vs[j].w = (kbase + 16 * j + 3 < L) ? pr.vs[j].w : 0u;
      }
    } else if constexpr (F16PAIR) {
      // word d of a uint4 holding key tiles kt0, kt0 + 1: keys 16 (kt0 + d/2) + 4 q4 + 2 (d%2) + {0, 1}
#pragma unroll
      for (int j = 0; j < PageRegs<D, FMT>::VSN; ++j) {
        const int kt0 = (FMT == 0) ? 2 * j : 2 * (j % 2);
        uint32_t mw[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int key = kbase + 16 * (kt0 + d / 2) + 2 * (d % 2);
          mw[d] = ((key < L) ? 0x0000FFFFu : 0u) | ((key + 1 < L) ? 0xFFFF0000u : 0u);
        }
        pr.vs[j].x &= mw[0];
        pr.vs[j].y &= mw[1];
        pr.vs[j].z &= mw[2];
        pr.vs[j].w &= mw[3];
      }
    }
  };
  // the largest V scale of this wave's share of page pr -> lower vexp if it asks for less;
  // returns whether it did, with f the factor the accumulators (and, for FP8, the row sums)
  // must be scaled by
  // (a vote on each lane's own largest scale against vth; the wave's largest is only
  // taken when some scale asks for a lower exponent, about once per chunk)
  auto lower_vexp = [&](PageRegs<D, FMT> &pr, float &f) -> bool {
    constexpr int NW4 = 4 * PageRegs<D, FMT>::VSN;
    uint32_t w[NW4];
#pragma unroll
    for (int j = 0; j < PageRegs<D, FMT>::VSN; ++j) {
      w[4 * j] = pr.vs[j].x;
      w[4 * j + 1] = pr.vs[j].y;
      w[4 * j + 2] = pr.vs[j].z;
      w[4 * j + 3] = pr.vs[j].w;
    }
    const uint32_t lm = (FMT == 1) ? lane_max_f32_scales(w) : lane_max_f16_scales(w);
    if (!__any(lm >= vth)) return false;
    const uint32_t wm = wave_max_u32(lm);
    const int E = (FMT == 1) ? scale_exponent_f32(wm) : scale_exponent_f16(wm);
    const int cur = __builtin_amdgcn_readfirstlane(vexp);
    if (E >= cur) return false;
    vexp = E;
    vth = __builtin_amdgcn_readfirstlane((FMT == 1) ? lower_threshold_f32(E) : lower_threshold_f16(E));
    if constexpr (F16PAIR) e2bits = __builtin_amdgcn_readfirstlane(f16x2_pow2(E));
    f = __builtin_ldexpf(1.0f, E - cur);
    return true;
  };
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m[nt] = -INFINITY;
    lsum[nt] = 0.0f;
    const int r = row0 + 16 * nt + c16;
    last[nt] = (r < R) ? (L - a.T + r / a.group) : -1;  // -1: padding row, sees nothing
    // the row's scores take back the 2^-s its query was scaled by (none for the BF16 pool)
    qsc[nt] = (FMT == 4) ? a.qk_scale_log2 : __builtin_ldexpf(a.qk_scale_log2, q_row_exp(
        (FMT == 2 || FMT == 3) ? __float_as_uint(__uint_as_float(lds_qmax[16 * nt + c16]) * 0.125f) : lds_qmax[16 * nt + c16]));
#pragma unroll
    for (int j = 0; j < DPW; ++j) o[nt][j] = f32x4{0, 0, 0, 0};
  }
  // ---- phase 1: scores of this wave's 16 keys (S^T = K Q^T), in log2 units, and their row maxima
  auto scores = [&](auto masked_tag, PageRegs<D, FMT> &pr, int p, float (&z)[NT][4], float (&mloc)[NT]) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int key0 = p * kPage + 16 * wave + 4 * q4;  // key of i is key0 + i
    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      acc[nt] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) z[nt][i] = 0.0f;
    }
    // the query fragments of 64-dim group cg, read from LDS two groups ahead of their use
    // (bf16 queries; fp32 queries, with twice the fragments, read them at their use)
    constexpr int QPF = (QLO || NT > 2) ? 1 : 2;  // groups of fragments in flight
    f16x8 qf[QPF][2][NT][QP];
    auto read_q = [&](f16x8 (&dst)[2][NT][QP], int cg) {
#pragma unroll
      for (int hk = 0; hk < 2; ++hk)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int hl = 0; hl < QP; ++hl) dst[hk][nt][hl] = lds_f16x8(&qs[(((nt * G64 + cg) * 2 + hk) * QP + hl) * 64 + lane]);
    };
#pragma unroll
    for (int c = 0; c < QPF && c < G64; ++c) read_q(qf[c], c);
#pragma unroll
    for (int cg = 0; cg < G64; ++cg) {
      f16x8 (&qc)[2][NT][QP] = qf[cg % QPF];
      if constexpr (QPF == 1) {
        if (cg > 0) read_q(qc, cg);
      }
#pragma unroll
      for (int hk = 0; hk < 2; ++hk) {
        if constexpr (FMT == 4) {  // bf16 keys enter the matrix cores as they are
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            acc[nt] = mfma16_bf(pr.k[2 * cg + hk], __builtin_bit_cast(uint4, qc[hk][nt][0]), acc[nt]);
            if constexpr (QLO) acc[nt] = mfma16_bf(pr.k[2 * cg + hk], __builtin_bit_cast(uint4, qc[hk][nt][QP - 1]), acc[nt]);
          }
          continue;
        }
        f16x8 ka;
        if constexpr (FMT == 3) {
          const uint4 &kw = pr.k[cg / 2];
          ka = k4_to_f16((cg & 1) ? (hk ? kw.w : kw.z) : (hk ? kw.y : kw.x));
        } else {
          ka = hk ? codes_to_f16<KF>(pr.k[cg].z, pr.k[cg].w) : codes_to_f16<KF>(pr.k[cg].x, pr.k[cg].y);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc[nt] = mfma16(ka, qc[hk][nt][0], acc[nt]);
          if constexpr (QLO) acc[nt] = mfma16(ka, qc[hk][nt][QP - 1], acc[nt]);
        }
      }
      if constexpr (QPF == 2) {
        if (cg + 2 < G64) read_q(qc, cg + 2);
      }
      if constexpr (KF != 1 && KF != 4) {  // fold each key's fp16 group scale, restart the group sum
        const uint4 w = pr.ks[cg >> 1];
        float sk[4];
        f16x2_to_f32((cg & 1) ? w.z : w.x, sk[0], sk[1]);
        f16x2_to_f32((cg & 1) ? w.w : w.y, sk[2], sk[3]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) z[nt][i] += sk[i] * acc[nt][i];
          acc[nt] = f32x4{0, 0, 0, 0};
        }
      }
    }
    if constexpr (FMT == 4) {  // no scales
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) z[nt][i] = acc[nt][i];
    }
    if constexpr (FMT == 1) {
      const float sk[4] = {__uint_as_float(pr.ks[0].x), __uint_as_float(pr.ks[0].y), __uint_as_float(pr.ks[0].z),
                           __uint_as_float(pr.ks[0].w)};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) z[nt][i] = sk[i] * acc[nt][i];
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = z[nt][i] * qsc[nt];
        if constexpr (MASKED) v = (key0 + i <= last[nt]) ? v : -INFINITY;
        z[nt][i] = v;
        mx = fmaxf(mx, v);
      }
      mloc[nt] = max_xor32(max_xor16(mx));
    }
  };

  // ---- phase 3: O^T += V^T P^T for this wave's dim tiles; each key's V scale folded into its weight
  auto accumulate = [&](auto masked_tag, PageRegs<D, FMT> &pr, int p, const float *pb) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    if constexpr (FMT == 4) {
      // BF16 pool: V^T straight from the pool (pr.v[2j + ks]: keys 16(2ks) + 4(lane/16) + i,
      // then 16(2ks+1) + ...), the fp32 weights as three bf16 terms
      if constexpr (MASKED) {  // slots at or past L may hold anything: zero their values
        const int kbase = p * kPage + 4 * q4;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          uint32_t mw[4];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int key = kbase + 16 * (2 * ks + w / 2) + 2 * (w % 2);
            mw[w] = ((key < L) ? 0x0000FFFFu : 0u) | ((key + 1 < L) ? 0xFFFF0000u : 0u);
          }
#pragma unroll
          for (int j = 0; j < DPW; ++j) {
            pr.v[2 * j + ks].x &= mw[0];
            pr.v[2 * j + ks].y &= mw[1];
            pr.v[2 * j + ks].z &= mw[2];
            pr.v[2 * j + ks].w &= mw[3];
          }
        }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float4 p0 = *reinterpret_cast<const float4 *>(pb + (16 * nt + c16) * PST + 16 * (2 * ks) + 4 * q4);
          const float4 p1 = *reinterpret_cast<const float4 *>(pb + (16 * nt + c16) * PST + 16 * (2 * ks + 1) + 4 * q4);
          uint32_t h[4], m[4], l[4];
          split_bf16x3(p0.x, p0.y, h[0], m[0], l[0]);
          split_bf16x3(p0.z, p0.w, h[1], m[1], l[1]);
          split_bf16x3(p1.x, p1.y, h[2], m[2], l[2]);
          split_bf16x3(p1.z, p1.w, h[3], m[3], l[3]);
          const uint4 bh = make_uint4(h[0], h[1], h[2], h[3]), bm = make_uint4(m[0], m[1], m[2], m[3]);
          const uint4 bl = make_uint4(l[0], l[1], l[2], l[3]);
#pragma unroll
          for (int j = 0; j < DPW; ++j) {
            o[nt][j] = mfma16_bf(pr.v[2 * j + ks], bh, o[nt][j]);
            o[nt][j] = mfma16_bf(pr.v[2 * j + ks], bm, o[nt][j]);
            o[nt][j] = mfma16_bf(pr.v[2 * j + ks], bl, o[nt][j]);
          }
        }
      return;
    }
    if constexpr (MASKED) {
      // slots at or past L may hold anything (never written): zero their V codes
      const int kbase = p * kPage + 4 * q4;  // key of (kt, i) is kbase + 16kt + i
      if constexpr (FMT >= 2) {
        // word ks holds keys kt = 2ks + q/4, i = q%4 (q = 0..7) at bit 16*(q%2) + 4*(q/2)
        uint32_t mw[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          uint32_t wv = 0;
#pragma unroll
          for (int q = 0; q < 8; ++q)
            wv |= (kbase + 16 * (2 * ks + q / 4) + q % 4 < L) ? (0xFu << (16 * (q % 2) + 4 * (q / 2))) : 0u;
          mw[ks] = wv;
        }
#pragma unroll
        for (int j = 0; j < PageRegs<D, FMT>::VN; ++j) {
          pr.v[j].x &= mw[0];
          pr.v[j].y &= mw[1];
          pr.v[j].z &= mw[0];
          pr.v[j].w &= mw[1];
        }
      } else {
        uint32_t mw[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          uint32_t wv = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) wv |= (kbase + 16 * kt + i < L) ? (0xFFu << (8 * i)) : 0u;
          mw[kt] = wv;
        }
#pragma unroll
        for (int j = 0; j < DPW; ++j) {
          pr.v[j].x &= mw[0];
          pr.v[j].y &= mw[1];
          pr.v[j].z &= mw[2];
          pr.v[j].w &= mw[3];
        }
      }
    }
    // the B operands (P^T, each key's weight times its V scale, as f16 hi + lo) of key
    // half ks; w: the fp16 V scales of keys 16(2ks) .. 16(2ks+1)+15 of this lane group
    auto build_b1 = [&](int ks, const uint4 &w, int nt, f16x8 &bh, f16x8 &bl) {
      {
        f16x2 hi[4], lo[4];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int kt = 2 * ks + kk;
          if constexpr (FMT != 1) {
            const uint4 pw = *reinterpret_cast<const uint4 *>(pb + (16 * nt + c16) * PST + 16 * kt + 4 * q4);
            const f16x2 h01 = __builtin_bit_cast(f16x2, pw.x), h23 = __builtin_bit_cast(f16x2, pw.y);
            const f16x2 l01 = __builtin_bit_cast(f16x2, pw.z), l23 = __builtin_bit_cast(f16x2, pw.w);
            f16x2 s01 = __builtin_bit_cast(f16x2, kk ? w.z : w.x), s23 = __builtin_bit_cast(f16x2, kk ? w.w : w.y);
            if constexpr (MASKED) {  // unwritten slots (weight 0) may hold NaN scales
              s01 = f16x2{h01[0] != _Float16(0) ? s01[0] : _Float16(0), h01[1] != _Float16(0) ? s01[1] : _Float16(0)};
              s23 = f16x2{h23[0] != _Float16(0) ? s23[0] : _Float16(0), h23[1] != _Float16(0) ? s23[1] : _Float16(0)};
            }
            scale_pair(h01, l01, s01, hi[2 * kk], lo[2 * kk]);
            scale_pair(h23, l23, s23, hi[2 * kk + 1], lo[2 * kk + 1]);
          } else {
            const float4 pw = *reinterpret_cast<const float4 *>(pb + (16 * nt + c16) * PST + 16 * kt + 4 * q4);
            const float pp[4] = {pw.x, pw.y, pw.z, pw.w};
            const uint4 sw = pr.vs[kt];
            const float sv[4] = {__uint_as_float(sw.x), __uint_as_float(sw.y), __uint_as_float(sw.z), __uint_as_float(sw.w)};
            float pv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              pv[i] = pp[i] * sv[i];
              if constexpr (MASKED) pv[i] = (pp[i] != 0.0f) ? pv[i] : 0.0f;  // unwritten slots: NaN scales
            }
            split_f16(pv[0], pv[1], hi[2 * kk], lo[2 * kk]);
            split_f16(pv[2], pv[3], hi[2 * kk + 1], lo[2 * kk + 1]);
          }
        }
        bh = f16x8{hi[0][0], hi[0][1], hi[1][0], hi[1][1], hi[2][0], hi[2][1], hi[3][0], hi[3][1]};
        bl = f16x8{lo[0][0], lo[0][1], lo[1][0], lo[1][1], lo[2][0], lo[2][1], lo[3][0], lo[3][1]};
      }
    };
    auto build_b = [&](int ks, const uint4 &w, f16x8 (&bh)[NT], f16x8 (&bl)[NT]) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) build_b1(ks, w, nt, bh[nt], bl[nt]);
    };
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if constexpr (FMT >= 2) {
        // one 32-dim scale group per pair of dim tiles, with its own B operands (built
        // one row tile at a time to keep few of them live)
#pragma unroll
        for (int gp = 0; gp < DPW / 2; ++gp) {
          const uint4 &vw = pr.v[gp];
          const f16x8 va0 = v4_to_f16(ks ? vw.y : vw.x), va1 = v4_to_f16(ks ? vw.w : vw.z);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            f16x8 bh, bl;
            build_b1(ks, pr.vs[2 * gp + ks], nt, bh, bl);
            o[nt][2 * gp] = mfma16(va0, bh, o[nt][2 * gp]);
            o[nt][2 * gp] = mfma16(va0, bl, o[nt][2 * gp]);
            o[nt][2 * gp + 1] = mfma16(va1, bh, o[nt][2 * gp + 1]);
            o[nt][2 * gp + 1] = mfma16(va1, bl, o[nt][2 * gp + 1]);
          }
        }
      } else {
        f16x8 bh[NT], bl[NT];
        build_b(ks, pr.vs[FMT == 0 ? ks : 0], bh, bl);
#pragma unroll
        for (int j = 0; j < DPW; ++j) {
          const f16x8 va = ks ? codes_to_f16<FMT>(pr.v[j].z, pr.v[j].w) : codes_to_f16<FMT>(pr.v[j].x, pr.v[j].y);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            o[nt][j] = mfma16(va, bh[nt], o[nt][j]);
            o[nt][j] = mfma16(va, bl[nt], o[nt][j]);
          }
        }
      }
    }
  };

  // one page: pr holds it; the next page's K half is already in flight in nx, and its
  // V half is issued once the page maxima are exchanged
  auto step = [&](PageRegs<D, FMT> &pr, PageRegs<D, FMT> &nx, int pg_next, int it, auto more_tag) {
    constexpr bool MORE = decltype(more_tag)::value;  // a next page exists: load its V half here
    const int p = page0 + it * NTEAM + team;
    const bool valid = p < page1;                              // uniform per team
    const bool full = (p * kPage + kPage - 1) <= lo_last;      // every real row sees every key of the page
    const int buf = it & 1;
    float z[NT][4];
    float mloc[NT];
    if (valid && full) {
      scores(std::false_type{}, pr, p, z, mloc);
    } else if (valid) {
      scores(std::true_type{}, pr, p, z, mloc);
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        mloc[nt] = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) z[nt][i] = -INFINITY;
      }
    }
    if (q4 == 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) reinterpret_cast<float *>(&lds_mx[team][buf][16 * nt + c16])[wave] = mloc[nt];
    }
    if constexpr (MORE) load_v_part<D, FMT>(nx, a, pg_next, wave, lane, q4);

    // ---- phase 2: softmax weights against the team's reference maxima m (one per row,
    // identical in the 4 waves).  m moves only when a page maximum passes it by more than
    // kLazy (log2 units), so weights stay <= 2^kLazy.  Each wave first assumes that no
    // maximum of the page passes m by that much and writes its weights with the current
    // m; if any wave of the workgroup saw such a maximum, all waves move m to the page
    // maxima exchanged beside the weights, rescale o and l, and rewrite their weights.
    float *pb = pbuf + (team * 2 + buf) * ROWS * PST;
    float psum[NT];
    auto write_weights = [&]() {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int r = 16 * nt + c16;
        const float mref = ((m[nt] == -INFINITY) ? 0.0f : m[nt]) - wexp();  // weights carry 2^wexp
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = exp2_hw(z[nt][i] - mref);
        psum[nt] = (pv[0] + pv[1]) + (pv[2] + pv[3]);
        if constexpr (FMT != 1 && FMT != 4) {
          // INT8 and rk8v4: the weights go out as f16 hi+lo pairs (the V scales, fp16, are
          // applied by the accumulating wave with packed f16 arithmetic)
          f16x2 h01, l01, h23, l23;
          split_f16(pv[0], pv[1], h01, l01);
          split_f16(pv[2], pv[3], h23, l23);
          *reinterpret_cast<uint4 *>(pb + r * PST + 16 * wave + 4 * q4) =
              make_uint4(__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23),
                         __builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23));
        } else {
          *reinterpret_cast<float4 *>(pb + r * PST + 16 * wave + 4 * q4) = make_float4(pv[0], pv[1], pv[2], pv[3]);
        }
      }
    };
    if constexpr (FMT == 1) {
      // FP8: the V-scale exponent rides on the weights, so it is settled before they are
      // written (all four waves of the team read the same 64 scales and agree on it)
      if (valid) {
        if (!full) zero_unwritten_scales(pr, p);
        float f;
        if (lower_vexp(pr, f)) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            lsum[nt] *= f;
#pragma unroll
            for (int j = 0; j < DPW; ++j) o[nt][j] *= f;
          }
        }
      }
    }
    bool over = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) over |= mloc[nt] > m[nt] + kLazy;  // m = -inf: any visible key
    const bool wave_over = __any(over);
    if (!wave_over) write_weights();  // a wave that is over rewrites below anyway
    if constexpr (F16PAIR) {
      // this wave's V-scale exponent: lowered (and o rescaled) if the page's scales ask for
      // it, then applied to the scales the products use; done while the other waves still
      // write their weights, so the chain stays off the path after the barrier
      if (valid) {
        if (!full) zero_unwritten_scales(pr, p);
        float f;
        if (lower_vexp(pr, f)) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int j = 0; j < DPW; ++j) o[nt][j] *= f;
        }
        const f16x2 e2 = __builtin_bit_cast(f16x2, e2bits);
#pragma unroll
        for (int j = 0; j < PageRegs<D, FMT>::VSN; ++j) {
          pr.vs[j].x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, pr.vs[j].x) * e2);
          pr.vs[j].y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, pr.vs[j].y) * e2);
          pr.vs[j].z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, pr.vs[j].z) * e2);
          pr.vs[j].w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, pr.vs[j].w) * e2);
        }
      }
    }
    if (lane == 0) lds_over[buf][(tid >> 6)] = wave_over ? 1 : 0;
    __syncthreads();
    int any_over = 0;
#pragma unroll
    for (int w = 0; w < 4 * NTEAM; ++w) any_over |= lds_over[buf][w];
    if (any_over) {  // uniform over the workgroup
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float4 mw4 = lds_mx[team][buf][16 * nt + c16];
        const float pmax = fmaxf(fmaxf(mw4.x, mw4.y), fmaxf(mw4.z, mw4.w));
        const bool up = pmax > m[nt] + kLazy;
        const float mnew = up ? pmax : m[nt];
        const float alpha = up ? exp2_hw(m[nt] - mnew) : 1.0f;  // 0 when m was -inf
        m[nt] = mnew;
        lsum[nt] *= alpha;
#pragma unroll
        for (int j = 0; j < DPW; ++j) o[nt][j] *= alpha;
      }
      write_weights();
      __syncthreads();
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) lsum[nt] += psum[nt];

    if constexpr (APP == 1) {
      if (defer && it == 0) {  // the deferred rows of the fused step (see above)
#pragma unroll
        for (int k = 0; k < RPW; ++k) {
          const int r = (tid >> 6) + k * NW;
          if (r < n_rows && blk_r[k] >= 0 && blk_r[k] < a.num_blocks)
            store_row<FMT, D>(aa, xr[k], kvh, r & 1, static_cast<long>(L) - a.T + t_lo + (r >> 1), blk_r[k], lane);
        }
      }
    }
    if (valid && full) {
      accumulate(std::false_type{}, pr, p, pb);
    } else if (valid) {
      accumulate(std::true_type{}, pr, p, pb);
    }
    if constexpr (APP == 1) {
      if (defer && it == 0 && (tid >> 6) < n_rows) __builtin_amdgcn_s_waitcnt(0);
    }
  };

  // pages in pairs while a next page exists for both; the last page (or two) peeled off
  // so that no load is issued past the team's pages
  int it = 0;
  for (; it + 2 < n_it; it += 2) {
    const int pgB = page_of(it + 1);
    load_k_part<D, FMT>(rB, a, pgB, wave, lane, q4);
    step(rA, rB, pgB, it, std::true_type{});
    const int pgA = page_of(it + 2);
    load_k_part<D, FMT>(rA, a, pgA, wave, lane, q4);
    step(rB, rA, pgA, it + 1, std::true_type{});
  }
  if (it + 1 < n_it) {
    const int pgB = page_of(it + 1);
    load_k_part<D, FMT>(rB, a, pgB, wave, lane, q4);
    step(rA, rB, pgB, it, std::true_type{});
    step(rB, rA, 0, it + 1, std::false_type{});
  } else if (it < n_it) {
    step(rA, rB, 0, it, std::false_type{});
  }

  // ---- per-wave row sums, then the team's and the workgroup's totals
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    lsum[nt] = sum_xor32(sum_xor16(lsum[nt]));
  }
  if (q4 == 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      lds_l[team][wave][16 * nt + c16] = lsum[nt];
      if (wave == 0) lds_m[team][16 * nt + c16] = m[nt] - wexp();  // the reference of l (and o)
    }
  }
  const int any_bad = __syncthreads_or(bad ? 1 : 0);
  float Mrow[NT], Lrow[NT], fown[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = 16 * nt + c16;
    float M = -INFINITY;
#pragma unroll
    for (int t = 0; t < NTEAM; ++t) M = fmaxf(M, lds_m[t][r]);
    const float Ms = (M == -INFINITY) ? 0.0f : M;
    float Lt = 0.0f;
#pragma unroll
    for (int t = 0; t < NTEAM; ++t) {
      const float lt = (lds_l[t][0][r] + lds_l[t][1][r]) + (lds_l[t][2][r] + lds_l[t][3][r]);
      Lt += lt * exp2f(lds_m[t][r] - Ms);
    }
    Mrow[nt] = M;
    Lrow[nt] = any_bad ? NAN : Lt;
    // this wave's o carries 2^(wexp + vexp) for the fp16-scale formats (l only 2^wexp)
    fown[nt] = exp2f(m[nt] - wexp() - Ms) * (F16PAIR ? __builtin_ldexpf(1.0f, -vexp) : 1.0f);
  }
  // teams 1.. hand their scaled outputs to team 0 through LDS (fixed order: deterministic)
  float *fin = pbuf;
  if constexpr (NTEAM > 1) {
    if (team > 0) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int j = 0; j < DPW; ++j) {
          const f32x4 v = o[nt][j] * fown[nt];
          *reinterpret_cast<float4 *>(fin + ((team - 1) * ROWS + 16 * nt + c16) * (D + 4) + 16 * (wave * DPW + j) +
                                      4 * q4) = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
    __syncthreads();
  }
  if (team == 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int rl = 16 * nt + c16, r = row0 + rl;
      if (r < R) {
        // one chunk per row block (or a one-chunk sequence of a balanced call): the
        // normalized row goes to out[b][t][h] (t*G + g = r)
        const size_t orow = ((static_cast<size_t>(b) * a.T + r / a.group) * a.num_q_heads + kvh * a.group +
                             r % a.group) * D;
#pragma unroll
        for (int j = 0; j < DPW; ++j) {
          f32x4 v = o[nt][j] * fown[nt];
          const int d = 16 * (wave * DPW + j) + 4 * q4;
#pragma unroll
          for (int t = 1; t < NTEAM; ++t) {
            const float4 x = *reinterpret_cast<const float4 *>(fin + ((t - 1) * ROWS + rl) * (D + 4) + d);
            v += f32x4{x.x, x.y, x.z, x.w};
          }
          if (direct) {
            const float l = Lrow[nt];
            *reinterpret_cast<float4 *>(a.out + orow + d) = make_float4(v[0] / l, v[1] / l, v[2] / l, v[3] / l);
          } else {
            *reinterpret_cast<float4 *>(a.ws_o + (part * R + r) * D + d) = make_float4(v[0], v[1], v[2], v[3]);
          }
        }
        if (!direct && wave == 0 && q4 == 0) {
          a.ws_ml[(part * R + r) * 2 + 0] = Mrow[nt];
          a.ws_ml[(part * R + r) * 2 + 1] = Lrow[nt];
        }
      }
    }
  }
}

// Merge kernel: MW waves per 64-dim slice of an output row (b, t, h).  Lane l of wave w
// holds float4 column l % 16 of the slice for the chunks s = 64 w + l / 16 + 4k (k < 16),
// with each chunk's maximum and sum; every load is issued at once, beside the sequence
// length.  Chunks beyond the first 64 MW come in further batches of 64 per wave, each
// batch issued at once.  All n_splits chunk slots lie in the workspace; slots past the
// chunks that hold the row's keys carry stale values and are dropped by selection.  The
// log-sum-exp weights and the sums over a wave's four chunk groups use cross-lane swaps;
// with MW > 1 the waves' maxima and sums meet in LDS, summed in wave order.  The order is
// fixed for a given MW (deterministic).  MW = 1 (no LDS, no barrier) serves calls of at
// most 64 chunks per (sequence, KV head), and balanced calls whatever their counts.
template <int D, int MW>
__global__ __launch_bounds__(64 * MW) void attn_merge_kernel(AttnArgs a) {
  constexpr int NQ = D / 64;       // 64-dim slices of a row
  constexpr int MPER = 16;         // chunks per lane and batch, held in registers
  constexpr int BATCH = 4 * MPER;  // chunks per wave and batch
  const int row = blockIdx.x / NQ, qs = blockIdx.x % NQ, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int h = row % a.num_q_heads, t = (row / a.num_q_heads) % a.T, b = row / (a.num_q_heads * a.T);
  float *dst = a.out + static_cast<size_t>(row) * D + 64 * qs;
  const int kvh = h / a.group, r = t * a.group + h % a.group;
  size_t part0 = (static_cast<size_t>(b) * a.num_kv_heads + kvh) * a.n_splits;  // slot of chunk 0
  int nsl = a.n_splits, tps = a.tokens_per_split;  // chunk slots of this (sequence, KV head), chunk length
  if (a.balanced != 0) {
    const BalancedChunks c = balanced_chunks(a, lane);
    nsl = __shfl(c.n, b);
    part0 = static_cast<size_t>(__shfl(c.first, b)) + static_cast<size_t>(kvh) * nsl;
    tps = c.tps;
    if (a.direct_single != 0 && nsl == 1) {  // the split workgroup wrote these rows itself
      const int L = a.seq_lens[b];
      if (w == 0 && (L < a.T || L > a.max_seq_len || L > static_cast<long>(a.max_blocks) * kPage)) dst[lane] = NAN;
      return;
    }
  }
  const int c4 = lane & 15, sg = lane >> 4, col = qs * 16 + c4;
  const float2 *ml2 = reinterpret_cast<const float2 *>(a.ws_ml);
  auto o_at = [&](int s) { return reinterpret_cast<const float4 *>(a.ws_o + ((part0 + s) * a.rows + r) * D)[col]; };

  float4 x[MPER];
  float2 ml[MPER];
#pragma unroll
  for (int k = 0; k < MPER; ++k) {
    const int s = min(BATCH * w + sg + 4 * k, nsl - 1);
    x[k] = o_at(s);
    ml[k] = ml2[(part0 + s) * a.rows + r];
  }
  const int L = a.seq_lens[b];
  if (L < a.T || L > a.max_seq_len || L > static_cast<long>(a.max_blocks) * kPage) {  // uniform per workgroup
    if (w == 0) dst[lane] = NAN;
    return;
  }
  // chunks holding keys this row sees (later chunks were skipped or hold none of them)
  const int ns = (L - a.T + t + tps) / tps;
  float mloc = -INFINITY;
#pragma unroll
  for (int k = 0; k < MPER; ++k)
    if (BATCH * w + sg + 4 * k < ns) mloc = fmaxf(mloc, ml[k].x);
  // later batches (few KV heads, long contexts): one memory latency per batch, not per chunk
  for (int s0 = BATCH * (w + MW); s0 < ns; s0 += BATCH * MW) {
    float mb[MPER];
#pragma unroll
    for (int k = 0; k < MPER; ++k) mb[k] = ml2[(part0 + min(s0 + sg + 4 * k, ns - 1)) * a.rows + r].x;
#pragma unroll
    for (int k = 0; k < MPER; ++k)
      if (s0 + sg + 4 * k < ns) mloc = fmaxf(mloc, mb[k]);
  }
  float M = max_xor32(max_xor16(mloc));
  __shared__ float red_m[MW], red_l[MW];
  __shared__ float4 red_acc[MW][16];
  if constexpr (MW > 1) {
    if (lane == 0) red_m[w] = M;
    __syncthreads();
    M = red_m[0];
#pragma unroll
    for (int i = 1; i < MW; ++i) M = fmaxf(M, red_m[i]);
  }
  const float Ms = (M == -INFINITY) ? 0.0f : M;
  float4 acc = make_float4(0, 0, 0, 0);
  float lt = 0.0f;
  auto add = [&](float2 st, float4 y) {
    const float wt = exp2f(st.x - Ms);
    lt += wt * st.y;
    acc.x += wt * y.x;
    acc.y += wt * y.y;
    acc.z += wt * y.z;
    acc.w += wt * y.w;
  };
#pragma unroll
  for (int k = 0; k < MPER; ++k)
    if (BATCH * w + sg + 4 * k < ns) add(ml[k], x[k]);
  for (int s0 = BATCH * (w + MW); s0 < ns; s0 += BATCH * MW) {  // the same batches, added in chunk order
#pragma unroll
    for (int k = 0; k < MPER; ++k) {
      const int s = min(s0 + sg + 4 * k, ns - 1);
      x[k] = o_at(s);
      ml[k] = ml2[(part0 + s) * a.rows + r];
    }
#pragma unroll
    for (int k = 0; k < MPER; ++k)
      if (s0 + sg + 4 * k < ns) add(ml[k], x[k]);
  }
  lt = sum_xor32(sum_xor16(lt));
  acc.x = sum_xor32(sum_xor16(acc.x));
  acc.y = sum_xor32(sum_xor16(acc.y));
  acc.z = sum_xor32(sum_xor16(acc.z));
  acc.w = sum_xor32(sum_xor16(acc.w));
  if constexpr (MW > 1) {
    if (sg == 0) red_acc[w][c4] = acc;
    if (lane == 0) red_l[w] = lt;
    __syncthreads();
    if (w != 0) return;
    acc = red_acc[0][c4];
    lt = red_l[0];
#pragma unroll
    for (int i = 1; i < MW; ++i) {
      const float4 o = red_acc[i][c4];
      acc.x += o.x;
      acc.y += o.y;
      acc.z += o.z;
      acc.w += o.w;
      lt += red_l[i];
    }
  }
  if (sg == 0) reinterpret_cast<float4 *>(dst)[c4] = make_float4(acc.x / lt, acc.y / lt, acc.z / lt, acc.w / lt);
}

// ---- Prefill kernel for INT8 and FP8 pools with bf16 queries.
//
// A workgroup of 8 waves owns 128 query rows (t*G + g) of one KV head and one chunk of
// its context; wave w owns rows 16w .. 16w+15 outright (KVQ_PREFILL_NTW = 2 builds 4
// waves of 32 rows instead, one wave per SIMD): their queries stay in registers
// as the B operands of S^T = K Q^T, their softmax state and their output O^T = V^T P^T
// (all D dims) stay in the wave, and the weights go from the score registers straight
// into the P·V products (the V layout puts each lane's keys where the S^T tile leaves
// them), so no wave waits on another for softmax.  The K and V codes of a page are
// converted to f16 once per workgroup, by all its threads, into LDS (double-buffered:
// page p+1 is converted while page p is multiplied, page p+2 is in flight from HBM), and
// every wave reads its matrix-core A operands from there: one barrier per page.
#ifndef KVQ_PREFILL_NTW
#define KVQ_PREFILL_NTW 1
#endif
template <int D, int FMT>
__global__ __launch_bounds__(64 * 8 / KVQ_PREFILL_NTW, 1) void prefill_kernel(AttnArgs a) {
  constexpr int G64 = D / 64, KB = D / 32, DT = D / 16, NTW = KVQ_PREFILL_NTW, ROWS = 128;
  constexpr int NW = 8 / NTW, NTH = 64 * NW;  // waves (16*NTW rows each) and threads of the workgroup
  constexpr int CPT = 64 * DT / NTH;          // 16-byte code chunks of K (and of V) per thread per page
  __shared__ uint4 kl[2][4 * KB * 64];  // f16 K operands: [(kt*KB + kb)*64 + lane]
  __shared__ uint4 vl[2][DT * 2 * 64];  // f16 V^T operands: [(dt*2 + ks)*64 + lane]
  // INT8: the page's K and V scales (D fp16 each), copied from the pool in its own layout,
  // so the waves read them from LDS (FP8 pools, one scale per key, read theirs directly)
  constexpr int SCU = (FMT == 0) ? D * 2 / 16 : 1;  // uint4 per scale array
  __shared__ uint4 sl[2][2 * SCU];
  // per buffer: the V-scale exponent in force from that page on (the running minimum of the
  // pages' exponents, see kWeightExp); every wave streams the same pages, so it is one
  // value for the workgroup, kept by wave 0, which converts the scales
  __shared__ int32_t sl_vexp[2];
  __shared__ int32_t lds_pg[kMaxPrefillChunkPages];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, q4 = lane >> 4, c16 = lane & 15;
  const int split = blockIdx.x, kvh = blockIdx.y % a.num_kv_heads, b = blockIdx.z;
  // row blocks last first: the later rows see the most keys (longest workgroups first)
  const int row0 = (a.row_blocks - 1 - static_cast<int>(blockIdx.y) / a.num_kv_heads) * ROWS;
  const int L = a.seq_lens[b];
  const int R = a.rows;
  if (L < a.T || L > a.max_seq_len || L > static_cast<long>(a.max_blocks) * kPage) {  // the merge writes NaN rows
    if (a.direct_out != 0 && split == 0) {                        // no merge: write them here
      for (int e = tid; e < ROWS * D; e += NTH) {
        const int r = row0 + e / D;
        if (r < R)
          a.out[((static_cast<size_t>(b) * a.T + r / a.group) * a.num_q_heads + kvh * a.group + r % a.group) * D +
                e % D] = NAN;
      }
    }
    return;
  }
  // keys the block's rows see: row r = t*G + g sees positions 0 .. L - T + t
  const int lim = L - a.T + (min(row0 + ROWS, R) - 1) / a.group + 1;
  const int lo_last = L - a.T + row0 / a.group;  // the last key the block's first row sees
  const int tok0 = split * a.tokens_per_split;
  if (tok0 >= lim) return;  // chunk past every key of these rows: the merge skips it
  const int tok1 = min(tok0 + a.tokens_per_split, lim);
  const int page0 = tok0 / kPage, npg = (tok1 + kPage - 1) / kPage - page0;

  // ---- the chunk's block ids -> pool pages in LDS (an invalid id reads block 0 and flags the chunk)
  bool bad = false;
  const int32_t *bt = a.block_table + static_cast<size_t>(b) * a.max_blocks;
  for (int i = tid; i < npg; i += NTH) {
    const int blk = bt[page0 + i];
    const bool ok = (blk >= 0) && (blk < a.num_blocks);
    bad |= !ok;
    lds_pg[i] = (ok ? blk : 0) * a.num_kv_heads + kvh;
  }
  const int any_bad = __syncthreads_or(bad ? 1 : 0);

  // ---- page codes: HBM -> registers -> f16 operands in LDS
  uint4 kc[CPT], vc[CPT], sc4 = make_uint4(0, 0, 0, 0);
  [[maybe_unused]] uint4 vs4 = make_uint4(0, 0, 0, 0);  // FP8: 16 threads hold the page's 64 V scales
  int cvexp = (FMT == 1) ? kFp8ExpMax : kVexpMax;       // wave 0: the exponent of the last converted page
  auto gload = [&](int i) {
    const size_t pg = static_cast<uint32_t>(lds_pg[i]);
    const uint4 *kp = reinterpret_cast<const uint4 *>(a.k_codes + pg * kPage * D);
    const uint4 *vp = reinterpret_cast<const uint4 *>(a.v_codes + pg * kPage * D);
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      kc[k] = ld_stream(kp + tid + NTH * k);
      vc[k] = ld_stream(vp + tid + NTH * k);
    }
    if constexpr (FMT == 0) {
      if (tid < 2 * SCU) {  // threads 0 .. SCU-1: K scales, SCU .. 2 SCU-1: V scales
        const uint4 *sp = reinterpret_cast<const uint4 *>(static_cast<const _Float16 *>(tid < SCU ? a.k_scales : a.v_scales) +
                                                          pg * D);
        sc4 = ld_stream(sp + (tid % SCU));
      }
    } else {
      if (tid < 16) vs4 = ld_stream(reinterpret_cast<const uint4 *>(static_cast<const float *>(a.v_scales) + pg * kPage) + tid);
    }
  };
  // wave 0: the page's largest V scale (slots at or past L skipped: they hold poison) sets the
  // V-scale exponent; INT8 scales go to LDS already multiplied by 2^exponent
  auto page_vexp = [&](int buf, int p) {
    uint32_t mx = 0;
    if constexpr (FMT == 0) {
      if (tid >= SCU && tid < 2 * SCU) {  // V-scale elements 8u .. 8u+7: (run * G64 + g) * 16 + pos
        const int u = tid - SCU, run = (8 * u / 16) / G64;
        const uint32_t w[4] = {sc4.x, sc4.y, sc4.z, sc4.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int pos = (8 * u + e) % 16, slot = 16 * (pos / 4) + 4 * run + pos % 4;
          const uint32_t h = (w[e / 2] >> (16 * (e % 2))) & 0xFFFFu;
          mx = (p * kPage + slot < L) ? max(mx, h) : mx;
        }
      }
    } else {
      if (tid < 16) {  // elements 4 tid + i: run tid / 4, pos 4 (tid % 4) + i
        const uint32_t w[4] = {vs4.x, vs4.y, vs4.z, vs4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int slot = 16 * (tid % 4) + 4 * (tid / 4) + i;
          mx = (p * kPage + slot < L) ? max(mx, w[i]) : mx;
        }
      }
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), o)));
    auto r = __builtin_amdgcn_permlane16_swap(mx, mx, false, false);
    mx = max(r[0], r[1]);
    r = __builtin_amdgcn_permlane32_swap(mx, mx, false, false);
    mx = max(r[0], r[1]);
    const int E = (FMT == 1) ? scale_exponent_f32(mx) : scale_exponent_f16(mx);
    cvexp = min(cvexp, E);
    if (lane == 0) sl_vexp[buf] = cvexp;
  };
  auto convert = [&](int buf, int p) {
    if (wave == 0) {
      page_vexp(buf, p);
      if constexpr (FMT == 0) {
        if (tid < SCU) {
          sl[buf][tid] = sc4;
        } else if (tid < 2 * SCU) {  // V scales times 2^cvexp (exact: a power of two, normal results)
          const f16x2 e2 = __builtin_bit_cast(f16x2, f16x2_pow2(cvexp));
          uint4 v = sc4;
          v.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, v.x) * e2);
          v.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, v.y) * e2);
          v.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, v.z) * e2);
          v.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, v.w) * e2);
          sl[buf][tid] = v;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int c = tid + NTH * k;
      // K chunk c: key s = (c / (16 DT)) * 16 + c % 16, dims 16 dt .. +15 with dt = (c / 16) % DT;
      // in the S^T products it is key tile s/16, dim block dt/2, lanes 16 (2 (dt%2) + hk) + s%16
      const int kt = c / (16 * DT), dt = (c / 16) % DT, sr = c % 16;
      uint4 *kd = &kl[buf][(kt * KB + dt / 2) * 64 + 32 * (dt % 2) + sr];
      kd[0] = __builtin_bit_cast(uint4, codes_to_f16<FMT>(kc[k].x, kc[k].y));
      kd[16] = __builtin_bit_cast(uint4, codes_to_f16<FMT>(kc[k].z, kc[k].w));
      // V chunk c: dim 16 (c/64) + c%16, the 16 keys 16 kt + 4 ((c%64)/16) + i; slots at or
      // past L may hold anything (never written): zero their codes
      uint4 v = vc[k];
      const int kbase = p * kPage + 4 * ((c % 64) / 16);
      if (kbase + 48 + 3 >= L) {
        uint32_t mw[4];
#pragma unroll
        for (int kt2 = 0; kt2 < 4; ++kt2) {
          uint32_t wv = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) wv |= (kbase + 16 * kt2 + i < L) ? (0xFFu << (8 * i)) : 0u;
          mw[kt2] = wv;
        }
        v.x &= mw[0];
        v.y &= mw[1];
        v.z &= mw[2];
        v.w &= mw[3];
      }
      vl[buf][((c / 64) * 2 + 0) * 64 + c % 64] = __builtin_bit_cast(uint4, codes_to_f16<FMT>(v.x, v.y));
      vl[buf][((c / 64) * 2 + 1) * 64 + c % 64] = __builtin_bit_cast(uint4, codes_to_f16<FMT>(v.z, v.w));
    }
  };
  if (npg > 0) gload(0);

  // ---- this wave's queries (bf16) -> registers: B operand of dim block kb.  Each row is
  // scaled by 2^-q_row_exp of its largest |element| (the four lane groups of a row share
  // it), which makes it exact in f16; the row's scores take the power of two back (qsc).
  f16x8 qf[NTW][KB];
  int last[NTW];
  float qsc[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int r = row0 + 16 * NTW * wave + 16 * nt + c16;
    last[nt] = (r < R) ? (L - a.T + r / a.group) : -1;  // -1: padding row, sees nothing
    const size_t qb = ((static_cast<size_t>(b) * a.T + r / a.group) * a.num_q_heads + kvh * a.group + r % a.group) * D;
    uint4 u[KB];
    uint32_t mx = 0;  // largest |element| of the row, bf16 bits
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      u[kb] = make_uint4(0, 0, 0, 0);
      if (r < R) u[kb] = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) + qb + 32 * kb + 8 * q4);
      const uint32_t w[4] = {u[kb].x, u[kb].y, u[kb].z, u[kb].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = max(mx, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
    }
    auto sw = __builtin_amdgcn_permlane16_swap(mx, mx, false, false);
    mx = max(sw[0], sw[1]);
    sw = __builtin_amdgcn_permlane32_swap(mx, mx, false, false);
    mx = max(sw[0], sw[1]);
    const int qe = q_row_exp(mx << 16);
    const float f = __builtin_ldexpf(1.0f, -qe);
    qsc[nt] = __builtin_ldexpf(a.qk_scale_log2, qe);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const uint32_t w[4] = {u[kb].x, u[kb].y, u[kb].z, u[kb].w};
      f16x2 h[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        h[j] = f16x2{static_cast<_Float16>(__uint_as_float(w[j] << 16) * f),
                     static_cast<_Float16>(__uint_as_float(w[j] & 0xFFFF0000u) * f)};
      qf[nt][kb] = f16x8{h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
    }
  }
  if (npg > 0) convert(0, page0);
  if (npg > 1) gload(1);
  __syncthreads();

  f32x4 o[NTW][DT];
  float m[NTW], lsum[NTW];
  // exponent offsets of the P·V operands (see kWeightExp): INT8 weights and row sums carry
  // 2^kWeightExp and o also the V-scale exponent vexp; FP8 weights, row sums and o carry vexp
  int vexp = (FMT == 1) ? kFp8ExpMax : kVexpMax;  // uniform over the workgroup
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    m[nt] = -INFINITY;
    lsum[nt] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[nt][dt] = f32x4{0, 0, 0, 0};
  }

  for (int it = 0; it < npg; ++it) {
    const int p = page0 + it, buf = it & 1;
    [[maybe_unused]] const size_t pg = static_cast<uint32_t>(lds_pg[it]);
    if (it + 1 < npg) convert(buf ^ 1, p + 1);  // the next page, loaded one iteration ago
    if (it + 2 < npg) gload(it + 2);
    const bool full = (p * kPage + kPage - 1) <= lo_last;  // every real row sees every key of the page
    {  // the page's V-scale exponent (set when it was converted): lower vexp, rescale if it moved
      const int E = __builtin_amdgcn_readfirstlane(sl_vexp[buf]);
      const int cur = __builtin_amdgcn_readfirstlane(vexp);
      if (E < cur) {
        const float f = __builtin_ldexpf(1.0f, E - cur);
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          if constexpr (FMT == 1) lsum[nt] *= f;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[nt][dt] *= f;
        }
        vexp = E;
      }
    }
    const float wexp = (FMT == 1) ? static_cast<float>(vexp) : static_cast<float>(kWeightExp);

    // ---- S^T = K Q^T for the 4 key tiles x this wave's 2 row tiles, scales folded per 64 dims
    float z[4][NTW][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) z[kt][nt][i] = 0.0f;
#pragma unroll
    for (int g = 0; g < G64; ++g) {
      f32x4 acc[4][NTW];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) acc[kt][nt] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int kb = 2 * g; kb < 2 * g + 2; ++kb)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const f16x8 ka = lds_f16x8(&kl[buf][(kt * KB + kb) * 64 + lane]);
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) acc[kt][nt] = mfma16(ka, qf[nt][kb], acc[kt][nt]);
        }
      if constexpr (FMT == 0) {
        // fp16 scales of this lane's keys 16 kt + 4 q4 + i in group g: element
        // ((q4*4 + kt) * G64 + g) * 4 + i of the page's K scales
        const uint2 *ksp = reinterpret_cast<const uint2 *>(&sl[buf][0]);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const uint2 w = ksp[(q4 * 4 + kt) * G64 + g];
          float sk[4];
          f16x2_to_f32(w.x, sk[0], sk[1]);
          f16x2_to_f32(w.y, sk[2], sk[3]);
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) z[kt][nt][i] += sk[i] * acc[kt][nt][i];
        }
      } else {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) z[kt][nt][i] += acc[kt][nt][i];
      }
    }
    if constexpr (FMT == 1) {  // one fp32 scale per key: element q4*16 + kt*4 + i
      const float4 *ksp = reinterpret_cast<const float4 *>(static_cast<const float *>(a.k_scales) + pg * kPage);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const float4 w = ksp[q4 * 4 + kt];
        const float sk[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) z[kt][nt][i] *= sk[i];
      }
    }
    // log2 units; the causal mask (and keys past L) on the pages that need it
    float pm[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = z[kt][nt][i] * qsc[nt];
          if (!full) v = (p * kPage + 16 * kt + 4 * q4 + i <= last[nt]) ? v : -INFINITY;
          z[kt][nt][i] = v;
          mx = fmaxf(mx, v);
        }
      pm[nt] = max_xor32(max_xor16(mx));
    }
    // ---- online softmax, per row inside the wave: the reference maximum moves only when
    // a page maximum passes it by more than kLazy (weights stay <= 2^kLazy)
    bool up = false;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) up |= pm[nt] > m[nt] + kLazy;
    if (__any(up)) {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const bool u = pm[nt] > m[nt] + kLazy;
        const float mnew = u ? pm[nt] : m[nt];
        const float alpha = u ? exp2_hw(m[nt] - mnew) : 1.0f;  // 0 when m was -inf
        m[nt] = mnew;
        lsum[nt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[nt][dt] *= alpha;
      }
    }
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const float ms = ((m[nt] == -INFINITY) ? 0.0f : m[nt]) - wexp;  // the weights carry 2^wexp
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          z[kt][nt][i] = exp2_hw(z[kt][nt][i] - ms);
          lsum[nt] += z[kt][nt][i];
        }
    }

    // ---- O^T += V^T P^T: key half ks is key tiles 2ks, 2ks+1 (this lane's keys 4 q4 + i of each)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if constexpr (FMT == 0) {
        f16x2 ph[NTW][4], pl[NTW][4];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            split_f16(z[2 * ks + kk][nt][0], z[2 * ks + kk][nt][1], ph[nt][2 * kk], pl[nt][2 * kk]);
            split_f16(z[2 * ks + kk][nt][2], z[2 * ks + kk][nt][3], ph[nt][2 * kk + 1], pl[nt][2 * kk + 1]);
          }
        // V scales (fp16) of this lane's keys in 64-dim group g: 8 values, element
        // (q4*G64 + g)*16 + 8 ks .. of the page's V scales
        const uint4 *vsp = &sl[buf][SCU];
#pragma unroll
        for (int g = 0; g < G64; ++g) {
          const uint4 w = vsp[(q4 * G64 + g) * 2 + ks];
          f16x2 sc[4] = {__builtin_bit_cast(f16x2, w.x), __builtin_bit_cast(f16x2, w.y), __builtin_bit_cast(f16x2, w.z),
                         __builtin_bit_cast(f16x2, w.w)};
          if (!full) {  // unwritten slots (weight 0) may hold NaN scales
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                const int key = p * kPage + 16 * (2 * ks + j / 2) + 4 * q4 + 2 * (j % 2) + e;
                if (key >= L) sc[j][e] = _Float16(0);
              }
          }
          f16x8 bh[NTW], bl[NTW];
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) {
            f16x2 hi[4], lo[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) scale_pair(ph[nt][j], pl[nt][j], sc[j], hi[j], lo[j]);
            bh[nt] = f16x8{hi[0][0], hi[0][1], hi[1][0], hi[1][1], hi[2][0], hi[2][1], hi[3][0], hi[3][1]};
            bl[nt] = f16x8{lo[0][0], lo[0][1], lo[1][0], lo[1][1], lo[2][0], lo[2][1], lo[3][0], lo[3][1]};
          }
#pragma unroll
          for (int dt = 4 * g; dt < 4 * g + 4; ++dt) {
            const f16x8 va = lds_f16x8(&vl[buf][(dt * 2 + ks) * 64 + lane]);
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt) {
              o[nt][dt] = mfma16(va, bh[nt], o[nt][dt]);
              o[nt][dt] = mfma16(va, bl[nt], o[nt][dt]);
            }
          }
        }
      } else {  // FP8: one fp32 scale per key, the same for every dim
        const float4 *vsp = reinterpret_cast<const float4 *>(static_cast<const float *>(a.v_scales) + pg * kPage);
        f16x8 bh[NTW], bl[NTW];
        float sv[2][4];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const float4 w = vsp[q4 * 4 + 2 * ks + kk];
          sv[kk][0] = w.x;
          sv[kk][1] = w.y;
          sv[kk][2] = w.z;
          sv[kk][3] = w.w;
        }
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          f16x2 hi[4], lo[4];
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            float pv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float pp = z[2 * ks + kk][nt][i];
              pv[i] = (pp != 0.0f) ? pp * sv[kk][i] : 0.0f;  // unwritten slots: NaN scales
            }
            split_f16(pv[0], pv[1], hi[2 * kk], lo[2 * kk]);
            split_f16(pv[2], pv[3], hi[2 * kk + 1], lo[2 * kk + 1]);
          }
          bh[nt] = f16x8{hi[0][0], hi[0][1], hi[1][0], hi[1][1], hi[2][0], hi[2][1], hi[3][0], hi[3][1]};
          bl[nt] = f16x8{lo[0][0], lo[0][1], lo[1][0], lo[1][1], lo[2][0], lo[2][1], lo[3][0], lo[3][1]};
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const f16x8 va = lds_f16x8(&vl[buf][(dt * 2 + ks) * 64 + lane]);
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) {
            o[nt][dt] = mfma16(va, bh[nt], o[nt][dt]);
            o[nt][dt] = mfma16(va, bl[nt], o[nt][dt]);
          }
        }
      }
    }
    __syncthreads();  // the next page's operands are in LDS; this page's buffer is free
  }

  // ---- rows: l summed over the 4 lanes of a row; normalized rows to out, or the partials.
  // The exponent offsets come out here: INT8 o carries 2^vexp more than l; the reference of
  // l (and o) is m - kWeightExp (INT8) or m - vexp (FP8).
  const float oscale = (FMT == 1) ? 1.0f : __builtin_ldexpf(1.0f, -vexp);
  const float wexp_end = (FMT == 1) ? static_cast<float>(vexp) : static_cast<float>(kWeightExp);
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const float lt = sum_xor32(sum_xor16(lsum[nt]));
    const int r = row0 + 16 * NTW * wave + 16 * nt + c16;
    if (r >= R) continue;
    const float l = any_bad ? NAN : lt;
    if (a.direct_out != 0) {
      const size_t orow = ((static_cast<size_t>(b) * a.T + r / a.group) * a.num_q_heads + kvh * a.group + r % a.group) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4 v = o[nt][dt] * oscale;
        *reinterpret_cast<float4 *>(a.out + orow + 16 * dt + 4 * q4) = make_float4(v[0] / l, v[1] / l, v[2] / l, v[3] / l);
      }
    } else {
      const size_t part = (static_cast<size_t>(b) * a.num_kv_heads + kvh) * a.n_splits + split;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4 v = o[nt][dt] * oscale;
        *reinterpret_cast<float4 *>(a.ws_o + (part * R + r) * D + 16 * dt + 4 * q4) = make_float4(v[0], v[1], v[2], v[3]);
      }
      if (q4 == 0) {
        a.ws_ml[(part * R + r) * 2 + 0] = m[nt] - wexp_end;
        a.ws_ml[(part * R + r) * 2 + 1] = l;
      }
    }
  }
}

template <int D, int NT, int FMT, int QDT>
hipError_t split_one(const AttnArgs &a, hipStream_t s) {
  // fp32 queries need the hi+lo pair; bf16 queries are one exact f16, unless rotated (rk8v4)
  constexpr int QLO = QDT == 0 ? 1 : ((FMT == 2 || FMT == 3) ? 2 : 0);
  const dim3 grid = a.balanced ? dim3(a.n_splits) : dim3(a.n_splits, a.num_kv_heads, a.num_seqs);
  if (a.k_new != nullptr)
    hipLaunchKernelGGL((attn_split_kernel<D, NT, FMT, QLO, kTeams, 1>), grid, dim3(256 * kTeams), 0, s, a);
  else
    hipLaunchKernelGGL((attn_split_kernel<D, NT, FMT, QLO, kTeams, 0>), grid, dim3(256 * kTeams), 0, s, a);
  return hipGetLastError();
}

template <int D, int FMT, int QDT>
hipError_t prefill_one(const AttnArgs &a, hipStream_t s) {
  if constexpr ((FMT == 0 || FMT == 1) && QDT == 1) {  // the prefill kernel: 128-row blocks
    const dim3 grid(a.n_splits, a.num_kv_heads * a.row_blocks, a.num_seqs);
    hipLaunchKernelGGL((prefill_kernel<D, FMT>), grid, dim3(64 * 8 / KVQ_PREFILL_NTW), 0, s, a);
    return hipGetLastError();
  }
  constexpr int QLO = QDT == 0 ? 1 : ((FMT == 2 || FMT == 3) ? 2 : 0);
  const dim3 grid(a.n_splits, a.num_kv_heads * a.row_blocks, a.num_seqs);
  hipLaunchKernelGGL((attn_split_kernel<D, kPrefillNT, FMT, QLO, kPrefillTeams, 2>), grid, dim3(256 * kPrefillTeams),
                     0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t merge_one(const AttnArgs &a, hipStream_t s) {
  const dim3 grid(a.num_seqs * a.T * a.num_q_heads * (D / 64));
  // more than 64 chunks per (sequence, KV head), as with one or two KV heads at long
  // contexts: 2 or 4 waves per slice.  (Balanced calls rarely exceed 64; the one-wave
  // kernel takes any count in batches.)
  const int chunks = a.balanced ? 0 : a.n_splits;
  if (chunks > 2 * 64)
    hipLaunchKernelGGL((attn_merge_kernel<D, 4>), grid, dim3(256), 0, s, a);
  else if (chunks > 64)
    hipLaunchKernelGGL((attn_merge_kernel<D, 2>), grid, dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL((attn_merge_kernel<D, 1>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

// The launches of one KV format (each format's kernels are compiled in a translation unit
// of their own, attn_f<FMT>.hip, so the library builds in parallel).
template <int F>
hipError_t split_fmt(int head_dim, int nt, int q_dtype, const AttnArgs &a, hipStream_t s) {
#define KVQ_SPLIT_CASE(DD, NTT, Q) \
  if (head_dim == DD && nt == NTT && q_dtype == Q) return split_one<DD, NTT, F, Q>(a, s);
  KVQ_SPLIT_CASE(128, 1, 0) KVQ_SPLIT_CASE(128, 1, 1) KVQ_SPLIT_CASE(128, 2, 0) KVQ_SPLIT_CASE(128, 2, 1)
  KVQ_SPLIT_CASE(256, 1, 0) KVQ_SPLIT_CASE(256, 1, 1) KVQ_SPLIT_CASE(256, 2, 0) KVQ_SPLIT_CASE(256, 2, 1)
#undef KVQ_SPLIT_CASE
  return hipErrorInvalidValue;
}

template <int F>
hipError_t prefill_fmt(int head_dim, int q_dtype, const AttnArgs &a, hipStream_t s) {
#define KVQ_PF_CASE(DD, Q) \
  if (head_dim == DD && q_dtype == Q) return prefill_one<DD, F, Q>(a, s);
  KVQ_PF_CASE(128, 0) KVQ_PF_CASE(128, 1) KVQ_PF_CASE(256, 0) KVQ_PF_CASE(256, 1)
#undef KVQ_PF_CASE
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace kvq

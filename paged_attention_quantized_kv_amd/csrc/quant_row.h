// quant_row.h -- quantize one K or V row of one KV head and write it into its
// page slot (the row quantizer of kv_append_quant, also run by the fused
// decode step).  One wave per row; each lane holds D/64 consecutive dims.
#pragma once

#include "internal.h"

namespace kvq {

template <int SRC>
__device__ inline float load_src(const void *p, size_t i);
template <>
__device__ inline float load_src<0>(const void *p, size_t i) {  // fp32
  return static_cast<const float *>(p)[i];
}
template <>
__device__ inline float load_src<1>(const void *p, size_t i) {  // bf16: exact widening
  return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(p)[i]) << 16);
}

// OCP FP8 E4M3FN of v, round to nearest even, magnitudes >= 448 saturate to
// 448, NaN -> 0x7F, sign kept (a negative value that rounds to zero -> 0x80).
// One branch-free form covers every range: with e = max(exponent of |v|, -6), the code
// is (e + 7) * 8 - 8 + rint(|v| * 2^(3 - e)), the significand in eighths for the normal
// codes and |v| in units of 2^-9 (the subnormal spacing) below 2^-6; a rounding that
// carries into the next binade lands on that binade's first code, and the minimum with
// 126 (448) saturates, infinities included.  The sum is exact below 2^24.
__device__ inline uint32_t e4m3fn_rne_sat(float v) {
  const uint32_t u = __float_as_uint(v), sign = (u >> 24) & 0x80u;
  const float ax = fabsf(v);
  const int e = max(static_cast<int>((u >> 23) & 0xFFu) - 127, -6);
  const float code = fminf(static_cast<float>((e + 7) * 8 - 8) + rintf(ldexpf(ax, 3 - e)), 126.0f);
  return (ax == ax) ? (sign | static_cast<uint32_t>(code)) : 0x7Fu;
}

// rk8v4 keys: the 64-dim groups of a key row are rotated by H64/8 (Sylvester-order
// Hadamard matrix, entry (j, i) = (-1)^popcount(i & j), over 8) before the INT8
// encoding (NInfer-3090 README, "RotorQuant KV (rk8v4)").  The butterflies run in
// binary64, where the sums of bf16 inputs are exact (unless a group's magnitudes
// span more than 2^39), and the result is rounded once to binary32.
//   x: the E consecutive elements (lane % (64/E)) * E + 0 .. E-1 of one 64-dim group,
//   which is spread over 64/E adjacent lanes.
template <int E>
__device__ inline void h64_rotate_lanes(float (&x)[E], int lane) {
  double y[E];
#pragma unroll
  for (int e = 0; e < E; ++e) y[e] = static_cast<double>(x[e]);
#pragma unroll
  for (int h = 1; h < E; h <<= 1)  // in-lane butterflies
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((e & h) == 0) {
        const double u = y[e], v = y[e + h];
        y[e] = u + v;
        y[e + h] = u - v;
      }
#pragma unroll
  for (int m = 1; m < 64 / E; m <<= 1) {  // across lanes: partner lane ^ m holds index ^ (m*E)
    const bool hi = (lane & m) != 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const double o = __shfl_xor(y[e], m);
      y[e] = hi ? (o - y[e]) : (y[e] + o);
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = static_cast<float>(y[e] * 0.125);
}

// rk8v4 values: bit offset (within the 4-byte-aligned word of a page of 64*D/2 bytes)
// of the 4-bit code of (slot s, dim d): see kvq.h.  Returns the word index and the shift.
__device__ inline void v4_place(int s, int d, size_t &word, int &shift) {
  const int r = (s % 16) / 4, j = s / 16, i = s % 4, dt = d / 16;
  const int k = (j % 2) * 4 + i;
  word = (static_cast<size_t>((dt / 2) * 64 + r * 16 + d % 16) * 16 + (dt % 2) * 8 + (j / 2) * 4) / 4;
  shift = 16 * (k % 2) + 4 * (k / 2);
}

// bfloat16 bits of v, round to nearest even (a carry may bump the exponent, up to
// infinity); NaN gives a quiet NaN.
__device__ inline uint32_t f32_to_bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// rk4v4 keys (NInfer-3090 README, "Lloyd-Max 4-bit keys (rk4v4)"): the INT8 codes of
// the 16 Lloyd-Max levels of a unit Gaussian, rint(127 * L_i / L_15), ascending; a
// rotated coordinate u = y / scale (the INT8 group scale) takes the level whose code is
// nearest, ties to the lower one: its index is the count of midpoints below u.
__device__ inline uint32_t rk4_index(float u) {
  constexpr float kMid[15] = {-111.5f, -85.5f, -66.5f, -51.0f, -37.5f, -24.5f, -12.0f, 0.0f,
                              12.0f,   24.5f,  37.5f,  51.0f,  66.5f,  85.5f,  111.5f};
  uint32_t k = 0;
#pragma unroll
  for (int m = 0; m < 15; ++m) k += (kMid[m] < u) ? 1u : 0u;
  return k;
}

// rk4v4 keys: byte offset of the 32-bit word holding dims 8*(d/8) .. +7 of slot s in a
// page of 64*D/2 bytes (see kvq.h); byte b of the word holds dim b (low nibble) and
// dim b + 4 (high nibble) of those 8.
template <int D>
__device__ inline size_t k4_word_byte(int s, int d) {
  const size_t unit = static_cast<size_t>((s / 16) * (D / 128) + d / 128) * 64 + ((d % 64) / 16) * 16 + (s % 16);
  return unit * 16 + ((d / 64) % 2) * 8 + ((d % 16) / 8) * 4;
}

// Row t of sequence b, KV head h, K (which=0) or V (which=1) of the
// [B][n_new][Hkv][D] source: this lane's D/64 consecutive elements, widened.
template <int D, int SRC>
__device__ inline void load_row(const AppendArgs &a, int b, int t, int h, int which, int lane, float (&x)[D / 64]) {
  constexpr int E = D / 64;
  const void *src = which ? a.v_new : a.k_new;
  const size_t base = ((static_cast<size_t>(b) * a.n_new + t) * a.num_kv_heads + h) * D + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = load_src<SRC>(src, base + e);
}

// Quantize a row held as x (D/64 elements per lane, see load_row) and store it
// at position pos of the sequence: slot pos % 64 of block blk, KV head h.
// Called by all 64 lanes of a wave.
template <int FMT, int D>
__device__ inline void store_row(const AppendArgs &a, const float (&xin)[D / 64], int h, int which, long pos, int blk,
                                 int lane) {
  constexpr int E = D / 64;            // elements per lane
  constexpr int LPG = 64 / E;          // lanes per 64-dim group
  const int slot = static_cast<int>(pos % kPage);
  const int run = (slot % 16) / 4, spos = (slot / 16) * 4 + slot % 4;
  float x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = xin[e];
  if constexpr (FMT == 2 || FMT == 3) {
    if (which == 0) h64_rotate_lanes<E>(x, lane);
  }

  const size_t page = static_cast<size_t>(blk) * a.num_kv_heads + h;
  uint32_t c[E];

  if constexpr (FMT == 4) {  // BF16: the element order of INT8 at two bytes per element
    uint16_t *el = reinterpret_cast<uint16_t *>(which ? a.v_codes : a.k_codes) + page * kPage * D;
    const int d0 = lane * E;
    if (which == 0) {  // the E dims of this lane are adjacent in one 16-dim tile row
      const size_t off = (static_cast<size_t>(slot / 16) * (D / 16) + d0 / 16) * 256 + (slot % 16) * 16 + d0 % 16;
      uint32_t wv[E / 2];
#pragma unroll
      for (int k = 0; k < E / 2; ++k) wv[k] = f32_to_bf16_rne(x[2 * k]) | (f32_to_bf16_rne(x[2 * k + 1]) << 16);
      if constexpr (E == 4) {
        *reinterpret_cast<uint2 *>(el + off) = make_uint2(wv[0], wv[1]);
      } else {
        *reinterpret_cast<uint32_t *>(el + off) = wv[0];
      }
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int d = d0 + e;
        el[(static_cast<size_t>(d / 16) * 4 + run) * 256 + (d % 16) * 16 + spos] = static_cast<uint16_t>(f32_to_bf16_rne(x[e]));
      }
    }
    return;
  }

  if constexpr (FMT == 3) {
    if (which == 0) {  // rk4v4 keys: level indices over the INT8 group scale of the rotated row
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
      for (int off = 1; off < LPG; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
      const _Float16 s16 = static_cast<_Float16>(amax / 127.0f);
      const float s = static_cast<float>(s16);
      // this lane's nibbles in the word of its 8-dim block; the 8/E lanes of a block
      // combine them and the first one writes the word (a row owns its key bytes)
      uint32_t wv = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int d = lane * E + e;
        wv |= rk4_index(s != 0.0f ? x[e] / s : 0.0f) << (8 * (d % 4) + 4 * ((d % 8) / 4));
      }
#pragma unroll
      for (int off = 1; off < 8 / E; off <<= 1) wv |= __shfl_xor(wv, off);
      if ((lane % (8 / E)) == 0)
        *reinterpret_cast<uint32_t *>(a.k_codes + page * kPage * (D / 2) + k4_word_byte<D>(slot, lane * E)) = wv;
      if ((lane % LPG) == 0) {
        const int g = lane / LPG;
        static_cast<_Float16 *>(a.k_scales)[page * D + ((run * 4 + slot / 16) * E + g) * 4 + slot % 4] = s16;
      }
      return;
    }
  }
  if constexpr (FMT == 2 || FMT == 3) {
    if (which == 1) {  // rk8v4 (and rk4v4) values: signed 4-bit codes, one fp16 scale per 32 dims
      constexpr int LPG32 = 32 / E;
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
      for (int off = 1; off < LPG32; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
      const _Float16 s16 = static_cast<_Float16>(amax / 7.0f);  // IEEE division, RNE to fp16
      const float s = static_cast<float>(s16);
      uint32_t *words = reinterpret_cast<uint32_t *>(a.v_codes + page * kPage * (D / 2));
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float r = 0.0f;
        if (s != 0.0f) r = fminf(fmaxf(rintf(x[e] / s), -7.0f), 7.0f);
        const uint32_t nib = static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xFu;
        size_t wi;
        int sh;
        v4_place(slot, lane * E + e, wi, sh);
        // other slots share the word (other rows of this launch may write them now)
        atomicAnd(words + wi, ~(0xFu << sh));
        atomicOr(words + wi, nib << sh);
      }
      if ((lane % LPG32) == 0) {
        const int g = lane / LPG32;
        static_cast<_Float16 *>(a.v_scales)[page * (kPage * D / 32) + (run * (D / 32) + g) * 16 + spos] = s16;
      }
      return;
    }
  }
  uint8_t *codes = (which ? a.v_codes : a.k_codes) + page * kPage * D;

  if constexpr (FMT == 0 || FMT == 2) {  // INT8 (rk8v4: of the rotated key), one fp16 scale per 64 dims
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
    for (int off = 1; off < LPG; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const _Float16 s16 = static_cast<_Float16>(amax / 127.0f);  // IEEE division, RNE to fp16
    const float s = static_cast<float>(s16);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float r = 0.0f;
      if (s != 0.0f) r = fminf(fmaxf(rintf(x[e] / s), -127.0f), 127.0f);
      c[e] = static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xFFu;
    }
    if ((lane % LPG) == 0) {
      const int g = lane / LPG;
      _Float16 *sc = static_cast<_Float16 *>(which ? a.v_scales : a.k_scales) + page * D;
      // K: (run, slot/16, group, slot%4); V: (run, group, slot/16, slot%4)
      const int e = which ? (run * E + g) * 16 + spos : ((run * 4 + slot / 16) * E + g) * 4 + slot % 4;
      sc[e] = s16;
    }
  } else {  // FP8 E4M3FN, one fp32 scale per row
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float s = amax / 448.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) c[e] = (s != 0.0f) ? e4m3fn_rne_sat(x[e] / s) : 0u;
    if (lane == 0) {
      float *sc = static_cast<float *>(which ? a.v_scales : a.k_scales) + page * kPage;
      sc[run * 16 + spos] = s;
    }
  }

  const int d0 = lane * E;
  if (which == 0) {
    // K: the E dims of this lane are adjacent bytes of one 16-byte tile row
    const size_t off = (static_cast<size_t>(slot / 16) * (D / 16) + d0 / 16) * 256 + (slot % 16) * 16 + d0 % 16;
    if constexpr (E == 4) {
      *reinterpret_cast<uint32_t *>(codes + off) = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    } else {
      *reinterpret_cast<uint16_t *>(codes + off) = static_cast<uint16_t>(c[0] | (c[1] << 8));
    }
  } else {
    // V: dim-major, one byte per dim
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int d = d0 + e;
      codes[(static_cast<size_t>(d / 16) * 4 + run) * 256 + (d % 16) * 16 + spos] = static_cast<uint8_t>(c[e]);
    }
  }
}

// load_row then store_row: row t of sequence b goes to position pos (block blk).
template <int FMT, int D, int SRC>
__device__ inline void quant_row(const AppendArgs &a, int b, int t, int h, int which, long pos, int blk, int lane) {
  float x[D / 64];
  load_row<D, SRC>(a, b, t, h, which, lane, x);
  store_row<FMT, D>(a, x, h, which, pos, blk, lane);
}

}  // namespace kvq

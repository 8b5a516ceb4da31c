// attn.hip -- paged decode attention over the quantized page pool.
//
// The result is out = softmax(q k^T * scale) v over the dequantized cache
// ("attention re-reads the whole cache each step": NInfer-3090 README,
// "Choosing a KV format"); the context of each (sequence, KV head) is cut into
// chunks (split-K over the context) whose partial results are merged with
// log-sum-exp weights.
//
// Split kernel: one workgroup = 4 independent waves on one chunk of one
// (sequence, KV head); the waves take the chunk's pages round-robin.  All
// T*G query rows of the KV head (T new tokens x G query heads of the group)
// ride along as the N dimension of 16x16x32 f16 matrix-core products, so every
// KV byte is read once:
//   S^T[key][row] = K[key][dim] * Q^T[dim][row]   (A = K codes, B = Q)
//   O^T[dim][row] = V^T[dim][key] * P^T[key][row] (A = V codes, B = softmax weights)
// K/V codes are converted to f16 exactly (int8 via byte permutes and one
// packed subtract, FP8 via the hardware converter); queries and softmax
// weights enter as f16 hi+lo pairs, so the only rounding is fp32 summation.
// The page layout (kvq.h) makes each 64-lane 16-byte load one contiguous KiB
// that lands in the operand registers with no LDS staging.
#include "internal.h"

namespace kvq {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));


__device__ inline f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
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

// x ~= hi + lo with hi = f16(x) rounded toward zero and lo = f16(x - hi): the
// pair carries ~21 significant bits.
__device__ inline void split_f16(float x0, float x1, f16x2 &hi, f16x2 &lo) {
  hi = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(x0, x1));
  lo = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(x0 - static_cast<float>(hi[0]),
                                                            x1 - static_cast<float>(hi[1])));
}

template <int QDT>
__device__ inline float load_q(const void *q, size_t i) {
  if constexpr (QDT == 1) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(q)[i]) << 16);
  return static_cast<const float *>(q)[i];
}

__device__ inline f16x8 lds_f16x8(const uint4 *p) { return __builtin_bit_cast(f16x8, *p); }

// Split kernel.  D: head_dim; NT: 16-row tiles of query rows (rows = T*G);
// FMT: 0 = INT8 g64, 1 = FP8 row; QDT: 0 = fp32 q, 1 = bf16 q.
template <int D, int NT, int FMT, int QDT>
__global__ __launch_bounds__(256, 1) void attn_split_kernel(AttnArgs a) {
  constexpr int G64 = D / 64;  // 64-dim groups
  constexpr int NCH = D / 16;  // 16-dim chunks (= output dim tiles)
  constexpr int ROWS = 16 * NT;
  constexpr int QS_U4 = NT * G64 * 2 * 2 * 64;          // Q operand entries (uint4)
  constexpr int O_STRIDE = D + 4;                        // padded LDS row of the merge buffer
  constexpr int O_FLOATS = ROWS * O_STRIDE;
  constexpr int SM_U4 = (QS_U4 * 4 > O_FLOATS ? QS_U4 * 4 : O_FLOATS) / 4;
  __shared__ uint4 smem[SM_U4];
  __shared__ float lds_m[kWaves][ROWS];
  __shared__ float lds_l[kWaves][ROWS];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q4 = lane >> 4, c16 = lane & 15;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int L = a.seq_lens[b];
  if (L < a.T || L > a.max_seq_len || L > a.max_blocks * kPage) return;  // merge writes NaN
  const int tok0 = split * a.tokens_per_split;
  if (tok0 >= L) return;  // chunk past the end of this sequence: the merge skips it
  const int tok1 = min(tok0 + a.tokens_per_split, L);
  const int page0 = tok0 / kPage, page1 = (tok1 + kPage - 1) / kPage;
  const int R = a.rows;

  // ---- queries -> LDS in B-operand order: entry (nt, cg, half, hl, lane) holds
  // dims 64cg + 16(lane/16) + 8half + 0..7 of row 16nt + lane%16, as f16 hi (hl=0) or lo (hl=1).
  for (int e = threadIdx.x; e < NT * G64 * 2 * 64; e += 256) {
    const int ln = e & 63, half = (e >> 6) & 1, cg = (e >> 7) % G64, nt = (e >> 7) / G64;
    const int r = 16 * nt + (ln & 15);
    const int d0 = 64 * cg + 16 * (ln >> 4) + 8 * half;
    f16x2 hi[4], lo[4];
    if (r < R) {
      const int t = r / a.group, h = kvh * a.group + r % a.group;
      const size_t qb = ((static_cast<size_t>(b) * a.T + t) * a.num_q_heads + h) * D + d0;
#pragma unroll
      for (int j = 0; j < 4; ++j) split_f16(load_q<QDT>(a.q, qb + 2 * j), load_q<QDT>(a.q, qb + 2 * j + 1), hi[j], lo[j]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) hi[j] = lo[j] = f16x2{0, 0};
    }
    const int idx = (((nt * G64 + cg) * 2 + half) * 2) * 64 + ln;
    smem[idx] = __builtin_bit_cast(uint4, f16x8{hi[0][0], hi[0][1], hi[1][0], hi[1][1], hi[2][0], hi[2][1], hi[3][0], hi[3][1]});
    smem[idx + 64] = __builtin_bit_cast(uint4, f16x8{lo[0][0], lo[0][1], lo[1][0], lo[1][1], lo[2][0], lo[2][1], lo[3][0], lo[3][1]});
  }
  __syncthreads();

  // Per-lane state: this lane's query row is 16nt + c16 in every tile.
  float m[NT], lsum[NT];
  f32x4 o[NT][NCH];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m[nt] = -INFINITY;
    lsum[nt] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < NCH; ++dt) o[nt][dt] = f32x4{0, 0, 0, 0};
  }
  // last visible key of this lane's row in each tile (-1: padding row, sees nothing)
  int last[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = 16 * nt + c16;
    last[nt] = (r < R) ? (L - a.T + r / a.group) : -1;
  }
  bool bad = false;

  for (int p = page0 + wave; p < page1; p += kWaves) {
    const int blk = a.block_table[static_cast<size_t>(b) * a.max_blocks + p];
    if (blk < 0 || blk >= a.num_blocks) {
      bad = true;
      continue;
    }
    const size_t pg = static_cast<size_t>(blk) * a.num_kv_heads + kvh;
    const uint4 *kp = reinterpret_cast<const uint4 *>(a.k_codes + pg * kPage * D);
    const uint4 *vp = reinterpret_cast<const uint4 *>(a.v_codes + pg * kPage * D);

    // ---- loads: K tile (kt, cg) and V dim tile dt are each one contiguous KiB
    uint4 kr[4][G64], vr[NCH];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int cg = 0; cg < G64; ++cg) kr[kt][cg] = kp[(kt * NCH + 4 * cg) * 16 + lane];
#pragma unroll
    for (int dt = 0; dt < NCH; ++dt) vr[dt] = vp[dt * 64 + lane];
    // scales of this lane group's 16 keys (key 16kt + 4q4 + i at position 4kt + i)
    uint4 ks[FMT == 0 ? G64 * 2 : 4], vs[FMT == 0 ? G64 * 2 : 4];
    if constexpr (FMT == 0) {
      const uint4 *ksp = reinterpret_cast<const uint4 *>(static_cast<const _Float16 *>(a.k_scales) + pg * D);
      const uint4 *vsp = reinterpret_cast<const uint4 *>(static_cast<const _Float16 *>(a.v_scales) + pg * D);
#pragma unroll
      for (int j = 0; j < G64 * 2; ++j) {
        ks[j] = ksp[q4 * G64 * 2 + j];
        vs[j] = vsp[q4 * G64 * 2 + j];
      }
    } else {
      const uint4 *ksp = reinterpret_cast<const uint4 *>(static_cast<const float *>(a.k_scales) + pg * kPage);
      const uint4 *vsp = reinterpret_cast<const uint4 *>(static_cast<const float *>(a.v_scales) + pg * kPage);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ks[j] = ksp[q4 * 4 + j];
        vs[j] = vsp[q4 * 4 + j];
      }
    }
    const int key0 = p * kPage + 4 * q4;  // key of (kt, i) is key0 + 16kt + i
    const bool full = (p * kPage + kPage - 1) <= (L - a.T);  // every real row sees every key

    if (!full) {
      // slots at or past L may hold anything (never written): zero their V codes
      uint32_t mw[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) w |= (key0 + 16 * kt + i < L) ? (0xFFu << (8 * i)) : 0u;
        mw[kt] = w;
      }
#pragma unroll
      for (int dt = 0; dt < NCH; ++dt) {
        vr[dt].x &= mw[0];
        vr[dt].y &= mw[1];
        vr[dt].z &= mw[2];
        vr[dt].w &= mw[3];
      }
    }

    // ---- S^T = K Q^T
    float z[NT][4][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) z[nt][kt][i] = 0.0f;
    f32x4 acc[NT][4];
#pragma unroll
    for (int cg = 0; cg < G64; ++cg) {
      if (FMT == 0 || cg == 0) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) acc[nt][kt] = f32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        f16x8 qh[NT], ql[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int idx = (((nt * G64 + cg) * 2 + half) * 2) * 64 + lane;
          qh[nt] = lds_f16x8(&smem[idx]);
          ql[nt] = lds_f16x8(&smem[idx + 64]);
        }
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const f16x8 ka = half ? codes_to_f16<FMT>(kr[kt][cg].z, kr[kt][cg].w) : codes_to_f16<FMT>(kr[kt][cg].x, kr[kt][cg].y);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            acc[nt][kt] = mfma16(ka, qh[nt], acc[nt][kt]);
            acc[nt][kt] = mfma16(ka, ql[nt], acc[nt][kt]);
          }
        }
      }
      if constexpr (FMT == 0) {
        // fold the fp16 group scale of each key
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const uint4 sw = ks[cg * 2 + (kt >> 1)];
          const uint32_t s01 = (kt & 1) ? sw.z : sw.x, s23 = (kt & 1) ? sw.w : sw.y;
          const f16x2 sa = __builtin_bit_cast(f16x2, s01), sb = __builtin_bit_cast(f16x2, s23);
          const float sk[4] = {static_cast<float>(sa[0]), static_cast<float>(sa[1]), static_cast<float>(sb[0]),
                               static_cast<float>(sb[1])};
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) z[nt][kt][i] += sk[i] * acc[nt][kt][i];
        }
      }
    }
    if constexpr (FMT == 1) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const uint4 sw = ks[kt];
        const float sk[4] = {__uint_as_float(sw.x), __uint_as_float(sw.y), __uint_as_float(sw.z), __uint_as_float(sw.w)};
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) z[nt][kt][i] = sk[i] * acc[nt][kt][i];
      }
    }

    // ---- online softmax (log2 domain), per row = per lane column
    float pw[NT][4][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = z[nt][kt][i] * a.qk_scale_log2;
          if (!full) v = (key0 + 16 * kt + i <= last[nt]) ? v : -INFINITY;
          z[nt][kt][i] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m[nt], mx);
      const float msafe = (mnew == -INFINITY) ? 0.0f : mnew;
      const float alpha = exp2f(m[nt] - msafe);
      m[nt] = mnew;
      float ps = 0.0f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pw[nt][kt][i] = exp2f(z[nt][kt][i] - msafe);
          ps += pw[nt][kt][i];
        }
      lsum[nt] = lsum[nt] * alpha + ps;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int dt = 0; dt < NCH; ++dt) o[nt][dt] *= alpha;
      }
    }

    // ---- O^T += V^T P^T, with each key's V scale folded into its weight
#pragma unroll
    for (int cg = 0; cg < G64; ++cg) {
      f16x8 bh[NT][2], bl[NT][2];
      if (FMT == 0 || cg == 0) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int ks2 = 0; ks2 < 2; ++ks2) {
            f16x2 h[4], l[4];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
              const int kt = 2 * ks2 + kk;
              float sv[4];
              if constexpr (FMT == 0) {
                const uint4 sw = vs[cg * 2 + (kt >> 1)];
                const uint32_t s01 = (kt & 1) ? sw.z : sw.x, s23 = (kt & 1) ? sw.w : sw.y;
                const f16x2 sa = __builtin_bit_cast(f16x2, s01), sb = __builtin_bit_cast(f16x2, s23);
                sv[0] = static_cast<float>(sa[0]);
                sv[1] = static_cast<float>(sa[1]);
                sv[2] = static_cast<float>(sb[0]);
                sv[3] = static_cast<float>(sb[1]);
              } else {
                const uint4 sw = vs[kt];
                sv[0] = __uint_as_float(sw.x);
                sv[1] = __uint_as_float(sw.y);
                sv[2] = __uint_as_float(sw.z);
                sv[3] = __uint_as_float(sw.w);
              }
              float pv[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                pv[i] = pw[nt][kt][i] * sv[i];
                if (!full) pv[i] = (pw[nt][kt][i] != 0.0f) ? pv[i] : 0.0f;  // unwritten slots: NaN scales
              }
              split_f16(pv[0], pv[1], h[2 * kk], l[2 * kk]);
              split_f16(pv[2], pv[3], h[2 * kk + 1], l[2 * kk + 1]);
            }
            bh[nt][ks2] = f16x8{h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
            bl[nt][ks2] = f16x8{l[0][0], l[0][1], l[1][0], l[1][1], l[2][0], l[2][1], l[3][0], l[3][1]};
          }
      }
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        const int dt = 4 * cg + dd;
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
          const f16x8 va = ks2 ? codes_to_f16<FMT>(vr[dt].z, vr[dt].w) : codes_to_f16<FMT>(vr[dt].x, vr[dt].y);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            o[nt][dt] = mfma16(va, bh[nt][ks2], o[nt][dt]);
            o[nt][dt] = mfma16(va, bl[nt][ks2], o[nt][dt]);
          }
        }
      }
    }
  }

  // ---- finish this wave: full running sum of each row
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    lsum[nt] += __shfl_xor(lsum[nt], 16);
    lsum[nt] += __shfl_xor(lsum[nt], 32);
  }

  // ---- merge the 4 waves of the workgroup (fixed order: deterministic)
  __syncthreads();  // Q operands no longer needed: smem becomes the merge buffer
  float *lds_o = reinterpret_cast<float *>(smem);
  if (q4 == 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      lds_m[wave][16 * nt + c16] = m[nt];
      lds_l[wave][16 * nt + c16] = lsum[nt];
    }
  }
  const int any_bad = __syncthreads_or(bad ? 1 : 0);
  float Mrow[NT], Lrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = 16 * nt + c16;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, lds_m[w][r]);
    const float Ms = (M == -INFINITY) ? 0.0f : M;
    float Lt = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) Lt += lds_l[w][r] * exp2f(lds_m[w][r] - Ms);
    Mrow[nt] = M;
    Lrow[nt] = any_bad ? NAN : Lt;
    const float f = exp2f(m[nt] - Ms);
#pragma unroll
    for (int dt = 0; dt < NCH; ++dt) o[nt][dt] *= f;
  }
  for (int w = 0; w < kWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int dt = 0; dt < NCH; ++dt) {
          float4 *dst = reinterpret_cast<float4 *>(lds_o + (16 * nt + c16) * O_STRIDE + 16 * dt + 4 * q4);
          float4 v = make_float4(o[nt][dt][0], o[nt][dt][1], o[nt][dt][2], o[nt][dt][3]);
          if (w != 0) {
            const float4 prev = *dst;
            v.x += prev.x;
            v.y += prev.y;
            v.z += prev.z;
            v.w += prev.w;
          }
          *dst = v;
        }
    }
    __syncthreads();
  }

  // ---- write this chunk's partial
  const size_t part = (static_cast<size_t>(b) * a.num_kv_heads + kvh) * a.n_splits + split;
  float *po = a.ws_o + part * R * D;
  for (int e = threadIdx.x; e < R * (D / 4); e += 256) {
    const int r = e / (D / 4), c4 = e % (D / 4);
    reinterpret_cast<float4 *>(po)[e] = *reinterpret_cast<const float4 *>(lds_o + r * O_STRIDE + 4 * c4);
  }
  if (wave == 0 && q4 == 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = 16 * nt + c16;
      if (r < R) {
        a.ws_ml[(part * R + r) * 2 + 0] = Mrow[nt];
        a.ws_ml[(part * R + r) * 2 + 1] = Lrow[nt];
      }
    }
  }
}

// Merge kernel: one workgroup per output row (b, t, h); thread d owns dim d.
template <int D>
__global__ __launch_bounds__(D) void attn_merge_kernel(AttnArgs a) {
  const int row = blockIdx.x;
  const int h = row % a.num_q_heads, t = (row / a.num_q_heads) % a.T, b = row / (a.num_q_heads * a.T);
  const int d = threadIdx.x;
  float *dst = a.out + static_cast<size_t>(row) * D + d;
  const int L = a.seq_lens[b];
  if (L < a.T || L > a.max_seq_len || L > a.max_blocks * kPage) {
    *dst = NAN;
    return;
  }
  const int kvh = h / a.group, r = t * a.group + h % a.group;
  const int ns = (L + a.tokens_per_split - 1) / a.tokens_per_split;
  const size_t part0 = (static_cast<size_t>(b) * a.num_kv_heads + kvh) * a.n_splits;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, a.ws_ml[((part0 + s) * a.rows + r) * 2]);
  const float Ms = (M == -INFINITY) ? 0.0f : M;
  float acc = 0.0f, lt = 0.0f;
  for (int s = 0; s < ns; ++s) {
    const size_t pr = (part0 + s) * a.rows + r;
    const float w = exp2f(a.ws_ml[pr * 2] - Ms);
    lt += w * a.ws_ml[pr * 2 + 1];
    acc += w * a.ws_o[pr * D + d];
  }
  *dst = acc / lt;
}

template <int D, int NT, int FMT, int QDT>
hipError_t split_one(const AttnArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((attn_split_kernel<D, NT, FMT, QDT>), dim3(a.n_splits, a.num_kv_heads, a.num_seqs), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

template <int D>
hipError_t merge_one(const AttnArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((attn_merge_kernel<D>), dim3(a.num_seqs * a.T * a.num_q_heads), dim3(D), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_split(int format, int head_dim, int q_dtype, const AttnArgs &a, hipStream_t s) {
  const int nt = (a.rows + 15) / 16;
#define KVQ_SPLIT_CASE(DD, NTT, F, Q) \
  if (head_dim == DD && nt == NTT && format == F && q_dtype == Q) return split_one<DD, NTT, F, Q>(a, s);
#define KVQ_SPLIT_DQ(DD, NTT) \
  KVQ_SPLIT_CASE(DD, NTT, 0, 0) KVQ_SPLIT_CASE(DD, NTT, 0, 1) KVQ_SPLIT_CASE(DD, NTT, 1, 0) KVQ_SPLIT_CASE(DD, NTT, 1, 1)
  KVQ_SPLIT_DQ(128, 1)
  KVQ_SPLIT_DQ(128, 2)
  KVQ_SPLIT_DQ(256, 1)
  KVQ_SPLIT_DQ(256, 2)
#undef KVQ_SPLIT_DQ
#undef KVQ_SPLIT_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_attn_merge(int head_dim, const AttnArgs &a, hipStream_t s) {
  if (head_dim == 128) return merge_one<128>(a, s);
  if (head_dim == 256) return merge_one<256>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace kvq

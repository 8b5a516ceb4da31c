// append.hip -- kv_append_quant: quantize new K/V rows on the way into the page
// pool; the append op is where KV quantization happens (NInfer-3090 README,
// intro and "RotorQuant KV (rk8v4)").
//
// One wave per (sequence, new row, KV head, K|V).  Each lane holds D/64
// consecutive dims, so a 64-dim group is 64/(D/64) adjacent lanes and its
// absmax is a butterfly over those lanes.  Codes go straight to their byte
// positions in the page (see kvq.h for the in-page order).
#include "quant_row.h"

namespace kvq {
namespace {

template <int FMT, int D, int SRC>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const long row = static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const long nrows = 2L * a.num_seqs * a.n_new * a.num_kv_heads;
  if (row >= nrows) return;
  const int which = static_cast<int>(row & 1);  // 0 = K, 1 = V
  long rest = row >> 1;
  const int h = static_cast<int>(rest % a.num_kv_heads);
  rest /= a.num_kv_heads;
  const int t = static_cast<int>(rest % a.n_new);
  const int b = static_cast<int>(rest / a.n_new);
  const long L0 = a.start_pos[b];
  if (a.start_back > 0 && (L0 < a.start_back || L0 > a.max_len || L0 > static_cast<long>(a.max_blocks) * kPage))
    return;
  const long pos = L0 - a.start_back + t;
  if (pos < 0 || pos >= static_cast<long>(a.max_blocks) * kPage) return;
  const int blk = a.block_table[static_cast<long>(b) * a.max_blocks + pos / kPage];
  if (blk < 0 || blk >= a.num_blocks) return;
  quant_row<FMT, D, SRC>(a, b, t, h, which, pos, blk, lane);
}

// rk8v4 keys in the bulk kernel: thread c16 holds dims 16*c16 .. +15 of its slot, so a
// 64-dim group is 4 neighbouring threads; in-thread butterflies, then two across threads
// (binary64, as in h64_rotate_lanes).
__device__ inline void h64_rotate_threads(float (&x)[16], int c16) {
  double y[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) y[e] = static_cast<double>(x[e]);
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if ((e & h) == 0) {
        const double u = y[e], v = y[e + h];
        y[e] = u + v;
        y[e + h] = u - v;
      }
#pragma unroll
  for (int m = 1; m < 4; m <<= 1) {
    const bool hi = (c16 & m) != 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const double o = __shfl_xor(y[e], m);
      y[e] = hi ? (o - y[e]) : (y[e] + o);
    }
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) x[e] = static_cast<float>(y[e] * 0.125);
}

// c[e] = rint(fl(x[e] / sc)) clamped to +-lim, as the row quantizer computes it, for the 16
// values of a thread whose quotients are bounded by lim (1 + 2^-11) < 128 (sc is the fp16
// scale of their group's maximum).  One division per thread instead of one per value:
// q0 = x * fl(1/sc) lies within 2^-23 |q| <= 2^-16 of q = x / sc, and fl(q) within 2^-18 of q,
// so rint(q0) is rint(fl(q)) whenever q0 is more than 2^-15 from a half-integer.  Only a
// thread holding a value that close divides its values out (about 2^-14 of values on random
// data, so a few percent of waves take that branch).
template <int LIM>
__device__ inline void rint_quotients(const float (&x)[16], float sc, uint32_t (&c)[16], uint32_t mask) {
  float r[16];
  const float rs = 1.0f / sc;
  bool amb = false;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float q0 = x[e] * rs;
    r[e] = rintf(q0);
    amb |= (0.5f - fabsf(q0 - r[e])) <= 0x1p-15f;
  }
  if (amb) {
#pragma unroll
    for (int e = 0; e < 16; ++e) r[e] = rintf(x[e] / sc);
  }
#pragma unroll
  for (int e = 0; e < 16; ++e)
    c[e] = static_cast<uint32_t>(static_cast<int32_t>(fminf(fmaxf(r[e], -static_cast<float>(LIM)), static_cast<float>(LIM)))) & mask;
}

// Bulk appends (prefill chunks): one workgroup per (page, KV head, K|V, sequence), one
// thread per (slot, 16 dims): 64 * D/16 threads.  Each thread quantizes its 16 values
// with the same arithmetic as quant_row (so the codes are identical), the group or row
// maximum coming from the neighbouring threads of the slot.  K codes leave as 16-byte
// tile rows (one slot each); V codes are staged in LDS and leave as 16-byte runs of the
// dim-major layout, or byte by byte on a page the chunk covers only in part.  Slots
// outside [start_pos, start_pos + n_new) are never written.
template <int FMT, int D, int SRC>
__global__ __launch_bounds__(kPage * D / 16) void append_page_kernel(AppendArgs a) {
  constexpr int NC = D / 16;  // threads per slot
  constexpr int G64 = D / 64;
  __shared__ __align__(16) uint8_t vstage[kPage * D * (FMT == 4 ? 2 : 1)];  // V codes, row-major [slot][dim]
  const int tid = threadIdx.x, sl = tid / NC, c16 = tid % NC;
  const int h = blockIdx.y, which = blockIdx.z & 1, b = blockIdx.z >> 1;
  const long pos0 = static_cast<long>(a.start_pos[b]) - a.start_back;
  if (pos0 < 0) return;
  const long pos_end = pos0 + a.n_new;           // exclusive
  const long pg = pos0 / kPage + blockIdx.x;
  if (pg * kPage >= pos_end || pg >= a.max_blocks) return;  // uniform per workgroup
  const int s_lo = static_cast<int>(max(pos0, pg * kPage) - pg * kPage);
  const int s_hi = static_cast<int>(min(pos_end, pg * kPage + kPage) - pg * kPage);
  const bool full = (s_lo == 0) && (s_hi == kPage);
  const bool mine = (sl >= s_lo) && (sl < s_hi);
  const int run = (sl % 16) / 4, spos = (sl / 16) * 4 + sl % 4;

  // ---- this thread's 16 source values (zeros for slots outside the chunk); the page's block
  // id is read after these loads are issued, so its latency overlaps theirs
  float x[16];
  if (mine) {
    const void *src = which ? a.v_new : a.k_new;
    const long row = pg * kPage + sl - pos0;
    const size_t base = ((static_cast<size_t>(b) * a.n_new + row) * a.num_kv_heads + h) * D + 16 * c16;
    if constexpr (SRC == 1) {  // bf16: two 16-byte loads, exact widening
      const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(src) + base);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint4 u = p[k];
        const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[8 * k + 2 * j] = __uint_as_float(wv[j] << 16);
          x[8 * k + 2 * j + 1] = __uint_as_float(wv[j] & 0xFFFF0000u);
        }
      }
    } else {  // fp32: four 16-byte loads
      const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(src) + base);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 f = p[k];
        x[4 * k] = f.x;
        x[4 * k + 1] = f.y;
        x[4 * k + 2] = f.z;
        x[4 * k + 3] = f.w;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) x[e] = 0.0f;
  }
  const int blk = a.block_table[static_cast<long>(b) * a.max_blocks + pg];
  if (blk < 0 || blk >= a.num_blocks) return;  // uniform per workgroup
  const size_t page = static_cast<size_t>(blk) * a.num_kv_heads + h;
  uint8_t *codes = (which ? a.v_codes : a.k_codes) + page * kPage * D;
  if constexpr (FMT == 4) {  // BF16: no quantization, the INT8 element order at two bytes each
    uint32_t hw[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) hw[k] = f32_to_bf16_rne(x[2 * k]) | (f32_to_bf16_rne(x[2 * k + 1]) << 16);
    if (which == 0) {  // the 16 dims of this slot: one 32-byte tile row
      if (mine) {
        uint4 *dst = reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(a.k_codes) + page * kPage * D +
                                               (static_cast<size_t>(sl / 16) * NC + c16) * 256 + (sl % 16) * 16);
        dst[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        dst[1] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
      }
      return;
    }
    uint16_t *vst = reinterpret_cast<uint16_t *>(vstage);
    uint4 *vrow = reinterpret_cast<uint4 *>(vst + sl * D + 16 * c16);
    vrow[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    vrow[1] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
    __syncthreads();
    // run k (one per thread): dim d = (k/64)*16 + k%16, run r = (k/16)%4; element 4j+i is slot 16j+4r+i
    const int k = tid, d = (k / 64) * 16 + (k % 16), r = (k / 16) % 4;
    uint16_t *dst = reinterpret_cast<uint16_t *>(a.v_codes) + page * kPage * D + static_cast<size_t>(k) * 16;
    if (full) {
      uint32_t v[8];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const int s0 = 16 * j + 4 * r + i;
          v[2 * j + i / 2] = static_cast<uint32_t>(vst[s0 * D + d]) | (static_cast<uint32_t>(vst[(s0 + 1) * D + d]) << 16);
        }
      reinterpret_cast<uint4 *>(dst)[0] = make_uint4(v[0], v[1], v[2], v[3]);
      reinterpret_cast<uint4 *>(dst)[1] = make_uint4(v[4], v[5], v[6], v[7]);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int sj = 16 * j + 4 * r + i;
          if (sj >= s_lo && sj < s_hi) dst[4 * j + i] = vst[sj * D + d];
        }
    }
    return;
  }
  if constexpr (FMT == 2 || FMT == 3) {
    if (which == 0) h64_rotate_threads(x, c16);  // rk8v4 / rk4v4 keys: rotate each 64-dim group
  }
  uint32_t c[16];
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(x[e]));
  if ((FMT == 2 || FMT == 3) && which == 1) {  // rk8v4 values: 4-bit codes, one fp16 scale per 32 dims (2 threads)
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    const _Float16 s16 = static_cast<_Float16>(amax / 7.0f);
    const float sc = static_cast<float>(s16);
    if (sc != 0.0f) {
      rint_quotients<7>(x, sc, c, 0xFu);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) c[e] = 0u;
    }
    if (mine && (c16 & 1) == 0)
      static_cast<_Float16 *>(a.v_scales)[page * (kPage * D / 32) + (run * (D / 32) + c16 / 2) * 16 + spos] = s16;
  } else if constexpr (FMT != 1) {  // INT8 (rk4v4: its scale), one fp16 scale per 64 dims: 4 neighbouring threads
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    const _Float16 s16 = static_cast<_Float16>(amax / 127.0f);
    const float sc = static_cast<float>(s16);
    if constexpr (FMT == 3) {  // rk4v4 key: the level index
#pragma unroll
      for (int e = 0; e < 16; ++e) c[e] = rk4_index(sc != 0.0f ? x[e] / sc : 0.0f);
    } else if (sc != 0.0f) {
      rint_quotients<127>(x, sc, c, 0xFFu);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) c[e] = 0u;
    }
    if (mine && (c16 & 3) == 0) {
      const int g = c16 / 4;
      _Float16 *scales = static_cast<_Float16 *>(which ? a.v_scales : a.k_scales) + page * D;
      scales[which ? (run * G64 + g) * 16 + spos : ((run * 4 + sl / 16) * G64 + g) * 4 + sl % 4] = s16;
    }
  } else {  // FP8 E4M3FN, one fp32 scale per row: the NC threads of the slot
#pragma unroll
    for (int off = 1; off < NC; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float sc = amax / 448.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) c[e] = (sc != 0.0f) ? e4m3fn_rne_sat(x[e] / sc) : 0u;
    if (mine && c16 == 0) static_cast<float *>(which ? a.v_scales : a.k_scales)[page * kPage + run * 16 + spos] = sc;
  }
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] = c[4 * k] | (c[4 * k + 1] << 8) | (c[4 * k + 2] << 16) | (c[4 * k + 3] << 24);

  if constexpr (FMT == 3) {
    if (which == 0) {  // rk4v4 K: the 16 level indices of this slot are its own 8 bytes
      if (mine) {
        uint32_t kw[2];
#pragma unroll
        for (int hk = 0; hk < 2; ++hk) {
          kw[hk] = 0;
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) kw[hk] |= (c[8 * hk + bb] << (8 * bb)) | (c[8 * hk + bb + 4] << (8 * bb + 4));
        }
        *reinterpret_cast<uint2 *>(a.k_codes + page * kPage * (D / 2) + k4_word_byte<D>(sl, 16 * c16)) =
            make_uint2(kw[0], kw[1]);
      }
      return;
    }
  }
  if (which == 0) {  // K: the 16 dims of this slot are one 16-byte tile row
    if (mine) {
      const size_t off = (static_cast<size_t>(sl / 16) * NC + c16) * 256 + (sl % 16) * 16;
      *reinterpret_cast<uint4 *>(codes + off) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    return;
  }
  // V: stage the page's codes row-major, then write the dim-major runs: run k (one per
  // thread) is dim d = (k/64)*16 + k%16, run r = (k/16)%4, whose byte 4j+i holds slot 16j+4r+i
  *reinterpret_cast<uint4 *>(vstage + sl * D + 16 * c16) = make_uint4(w[0], w[1], w[2], w[3]);
  __syncthreads();
  if constexpr (FMT == 2 || FMT == 3) {
    // rk8v4: 8-byte chunk k (one per thread) holds dim d = 16*dt + (k/2)%16 with
    // dt = 2*(k/128) + k%2, run r = (k/32)%4; its word w holds the slots 16*(2w + q/4) +
    // 4r + q%4 (q = 0..7), code q at bit 16*(q%2) + 4*(q/2)
    const int k = tid, dt = 2 * (k / 128) + (k % 2), d = 16 * dt + (k / 2) % 16, r = (k / 32) % 4;
    uint32_t *words = reinterpret_cast<uint32_t *>(a.v_codes + page * kPage * (D / 2)) + 2 * static_cast<size_t>(k);
    uint32_t v[2], m[2];
#pragma unroll
    for (int wv = 0; wv < 2; ++wv) {
      v[wv] = 0;
      m[wv] = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int sj = 16 * (2 * wv + q / 4) + 4 * r + q % 4;
        const int sh = 16 * (q % 2) + 4 * (q / 2);
        v[wv] |= static_cast<uint32_t>(vstage[sj * D + d]) << sh;
        if (sj >= s_lo && sj < s_hi) m[wv] |= 0xFu << sh;
      }
    }
    if (full) {
      *reinterpret_cast<uint2 *>(words) = make_uint2(v[0], v[1]);
    } else {  // keep the codes of slots outside the chunk (this thread owns the word)
#pragma unroll
      for (int wv = 0; wv < 2; ++wv)
        if (m[wv] != 0) words[wv] = (words[wv] & ~m[wv]) | (v[wv] & m[wv]);
    }
    return;
  }
  const int k = tid, d = (k / 64) * 16 + (k % 16), r = (k / 16) % 4;
  if (full) {
    uint32_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s0 = 16 * j + 4 * r;
      v[j] = static_cast<uint32_t>(vstage[s0 * D + d]) | (static_cast<uint32_t>(vstage[(s0 + 1) * D + d]) << 8) |
             (static_cast<uint32_t>(vstage[(s0 + 2) * D + d]) << 16) |
             (static_cast<uint32_t>(vstage[(s0 + 3) * D + d]) << 24);
    }
    *reinterpret_cast<uint4 *>(codes + static_cast<size_t>(k) * 16) = make_uint4(v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int sj = 16 * j + 4 * r + i;
        if (sj >= s_lo && sj < s_hi) codes[static_cast<size_t>(k) * 16 + 4 * j + i] = vstage[sj * D + d];
      }
  }
}

template <int FMT, int D, int SRC>
hipError_t launch_one(const AppendArgs &a, hipStream_t s) {
  if (a.n_new >= kBulkAppendRows) {
    // pages a chunk of n_new rows can touch, whatever its start
    const long pages = (a.n_new + kPage - 1) / kPage + 1;
    hipLaunchKernelGGL((append_page_kernel<FMT, D, SRC>), dim3(static_cast<unsigned>(pages), a.num_kv_heads,
                                                               2 * a.num_seqs), dim3(kPage * D / 16), 0, s, a);
    return hipGetLastError();
  }
  const long nrows = 2L * a.num_seqs * a.n_new * a.num_kv_heads;
  const long nblk = (nrows + 3) / 4;
  hipLaunchKernelGGL((append_kernel<FMT, D, SRC>), dim3(static_cast<unsigned>(nblk)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(int format, int head_dim, int src_dtype, const AppendArgs &a, hipStream_t s) {
  if (a.num_seqs == 0 || a.n_new == 0) return hipSuccess;
#define KVQ_APPEND_CASE(F, DD, S) \
  if (format == F && head_dim == DD && src_dtype == S) return launch_one<F, DD, S>(a, s);
  KVQ_APPEND_CASE(0, 128, 0)
  KVQ_APPEND_CASE(0, 128, 1)
  KVQ_APPEND_CASE(0, 256, 0)
  KVQ_APPEND_CASE(0, 256, 1)
  KVQ_APPEND_CASE(1, 128, 0)
  KVQ_APPEND_CASE(1, 128, 1)
  KVQ_APPEND_CASE(1, 256, 0)
  KVQ_APPEND_CASE(1, 256, 1)
  KVQ_APPEND_CASE(2, 128, 0)
  KVQ_APPEND_CASE(2, 128, 1)
  KVQ_APPEND_CASE(2, 256, 0)
  KVQ_APPEND_CASE(2, 256, 1)
  KVQ_APPEND_CASE(3, 128, 0)
  KVQ_APPEND_CASE(3, 128, 1)
  KVQ_APPEND_CASE(3, 256, 0)
  KVQ_APPEND_CASE(3, 256, 1)
  KVQ_APPEND_CASE(4, 128, 0)
  KVQ_APPEND_CASE(4, 128, 1)
  KVQ_APPEND_CASE(4, 256, 0)
  KVQ_APPEND_CASE(4, 256, 1)
#undef KVQ_APPEND_CASE
  return hipErrorInvalidValue;
}

}  // namespace kvq

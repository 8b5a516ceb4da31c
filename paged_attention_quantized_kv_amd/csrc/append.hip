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
  const long pos = static_cast<long>(a.start_pos[b]) + t;
  if (pos < 0 || pos >= static_cast<long>(a.max_blocks) * kPage) return;
  const int blk = a.block_table[static_cast<long>(b) * a.max_blocks + pos / kPage];
  if (blk < 0 || blk >= a.num_blocks) return;
  quant_row<FMT, D, SRC>(a, b, t, h, which, pos, blk, lane);
}

template <int FMT, int D, int SRC>
hipError_t launch_one(const AppendArgs &a, hipStream_t s) {
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
#undef KVQ_APPEND_CASE
  return hipErrorInvalidValue;
}

}  // namespace kvq

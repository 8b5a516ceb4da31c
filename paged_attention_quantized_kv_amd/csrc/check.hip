// check.hip -- kvq_check_tables: the debug checker of the device-resident tables whose
// values the other calls take as preconditions (sequence lengths and block ids).
#include "internal.h"

namespace kvq {
namespace {

// One workgroup walks every sequence and every block-table entry of the pages its
// length uses; counts go through LDS and are written once at the end.
__global__ __launch_bounds__(1024) void check_tables_kernel(CheckArgs a) {
  __shared__ int cnt[2];
  const int tid = threadIdx.x;
  if (tid < 2) cnt[tid] = 0;
  __syncthreads();
  for (int b = tid; b < a.num_seqs; b += 1024) {
    const int L = a.seq_lens[b];
    if (L < a.T || L > a.max_seq_len) atomicAdd(&cnt[0], 1);
  }
  const long n = static_cast<long>(a.num_seqs) * a.max_blocks;
  for (long i = tid; i < n; i += 1024) {
    const int b = static_cast<int>(i / a.max_blocks), p = static_cast<int>(i % a.max_blocks);
    const int L = min(max(a.seq_lens[b], 0), a.max_seq_len);
    if (p < (L + kPage - 1) / kPage) {
      const int blk = a.block_table[i];
      if (blk < 0 || blk >= a.num_blocks) atomicAdd(&cnt[1], 1);
    }
  }
  __syncthreads();
  if (tid < 2) a.result[tid] = cnt[tid];
}

}  // namespace

hipError_t launch_check_tables(const CheckArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(check_tables_kernel, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq

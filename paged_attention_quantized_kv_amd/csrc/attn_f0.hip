// attn_f0.hip -- the attention kernels of KV format 0 (kvq_format_t), one translation unit
// per format so the library compiles in parallel.
#include "attn_kernels.h"

namespace kvq {

hipError_t launch_attn_split_f0(int head_dim, int nt, int q_dtype, const AttnArgs &a, hipStream_t s) {
  return split_fmt<0>(head_dim, nt, q_dtype, a, s);
}

hipError_t launch_attn_prefill_f0(int head_dim, int q_dtype, const AttnArgs &a, hipStream_t s) {
  return prefill_fmt<0>(head_dim, q_dtype, a, s);
}

}  // namespace kvq

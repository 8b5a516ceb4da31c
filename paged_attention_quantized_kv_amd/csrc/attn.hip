// attn.hip -- dispatch of the attention launches by KV format, and the merge launch.
// The kernels live in attn_kernels.h; each format's instances are compiled in attn_f<FMT>.hip.
#include "attn_kernels.h"

namespace kvq {

hipError_t launch_attn_split_f0(int head_dim, int nt, int q_dtype, const AttnArgs &a, hipStream_t s);
hipError_t launch_attn_split_f1(int head_dim, int nt, int q_dtype, const AttnArgs &a, hipStream_t s);
hipError_t launch_attn_split_f2(int head_dim, int nt, int q_dtype, const AttnArgs &a, hipStream_t s);
hipError_t launch_attn_split_f3(int head_dim, int nt, int q_dtype, const AttnArgs &a, hipStream_t s);
hipError_t launch_attn_split_f4(int head_dim, int nt, int q_dtype, const AttnArgs &a, hipStream_t s);
hipError_t launch_attn_prefill_f0(int head_dim, int q_dtype, const AttnArgs &a, hipStream_t s);
hipError_t launch_attn_prefill_f1(int head_dim, int q_dtype, const AttnArgs &a, hipStream_t s);
hipError_t launch_attn_prefill_f2(int head_dim, int q_dtype, const AttnArgs &a, hipStream_t s);
hipError_t launch_attn_prefill_f3(int head_dim, int q_dtype, const AttnArgs &a, hipStream_t s);
hipError_t launch_attn_prefill_f4(int head_dim, int q_dtype, const AttnArgs &a, hipStream_t s);

hipError_t launch_attn_split(int format, int head_dim, int q_dtype, const AttnArgs &a, hipStream_t s) {
  const int nt = (a.rows + 15) / 16;
  switch (format) {
    case 0: return launch_attn_split_f0(head_dim, nt, q_dtype, a, s);
    case 1: return launch_attn_split_f1(head_dim, nt, q_dtype, a, s);
    case 2: return launch_attn_split_f2(head_dim, nt, q_dtype, a, s);
    case 3: return launch_attn_split_f3(head_dim, nt, q_dtype, a, s);
    case 4: return launch_attn_split_f4(head_dim, nt, q_dtype, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_prefill(int format, int head_dim, int q_dtype, const AttnArgs &a, hipStream_t s) {
  switch (format) {
    case 0: return launch_attn_prefill_f0(head_dim, q_dtype, a, s);
    case 1: return launch_attn_prefill_f1(head_dim, q_dtype, a, s);
    case 2: return launch_attn_prefill_f2(head_dim, q_dtype, a, s);
    case 3: return launch_attn_prefill_f3(head_dim, q_dtype, a, s);
    case 4: return launch_attn_prefill_f4(head_dim, q_dtype, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_merge(int head_dim, const AttnArgs &a, hipStream_t s) {
  if (head_dim == 128) return merge_one<128>(a, s);
  if (head_dim == 256) return merge_one<256>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace kvq

// internal.h -- shared declarations of the HIP library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "shape.h"

namespace kvq {

// Launch arguments of kv_append_quant, validated on the host.
struct AppendArgs {
  const void *k_new, *v_new;
  uint8_t *k_codes, *v_codes;
  void *k_scales, *v_scales;
  const int32_t *block_table;
  const int32_t *start_pos;
  int32_t start_back;  // sequence b's rows go to positions start_pos[b] - start_back + t
  int32_t max_len;     // start_back > 0 (start_pos = lengths): a length outside [start_back,
                       // min(max_len, max_blocks * 64)] skips the sequence, as the fused step does
  int32_t num_seqs, n_new, num_kv_heads, max_blocks, num_blocks;
};

// Launch arguments of the two attention phases, validated on the host.
struct AttnArgs {
  const uint8_t *k_codes, *v_codes;
  const void *k_scales, *v_scales;
  const void *q;
  const int32_t *block_table;
  const int32_t *seq_lens;
  float *ws_ml;  // [B][Hkv][n_splits][R][2]: running max (log2 units), running sum
  float *ws_o;   // [B][Hkv][n_splits][R][D]: unnormalized output
  float *out;    // [B][T][Hq][D]
  const void *k_new, *v_new;  // fused decode step: [B][T][Hkv][D] rows to append first (else null)
  int32_t num_seqs, num_blocks, num_kv_heads, num_q_heads, group, T, rows;
  int32_t max_blocks, max_seq_len, tokens_per_split, n_splits;
  int32_t row_blocks;   // blocks of 16*NT query rows per KV head (grid y = row_blocks * num_kv_heads)
  int32_t direct_out;   // one chunk per row block: write normalized rows to out, no merge
  float qk_scale_log2;  // softmax_scale * log2(e)
  // balanced != 0 (decode, 2..kMaxBalancedSeqs sequences): chunks of one common length set on
  // the device from the actual lengths (balanced_chunks); n_splits is then the number of
  // partial slots and split workgroups (grid x), not the chunks per (sequence, KV head)
  int32_t balanced;
  // balanced, one call: a sequence of one chunk writes its normalized rows and the merge
  // skips it
  int32_t direct_single;
};

// Launch arguments of kvq_check_tables, validated on the host.
struct CheckArgs {
  const int32_t *block_table;
  const int32_t *seq_lens;
  int32_t *result;
  int32_t num_seqs, T, max_blocks, max_seq_len, num_blocks;
};

hipError_t launch_check_tables(const CheckArgs &a, hipStream_t s);
hipError_t launch_append(int format, int head_dim, int src_dtype, const AppendArgs &a, hipStream_t s);
hipError_t launch_attn_split(int format, int head_dim, int q_dtype, const AttnArgs &a, hipStream_t s);
hipError_t launch_attn_merge(int head_dim, const AttnArgs &a, hipStream_t s);
hipError_t launch_attn_prefill(int format, int head_dim, int q_dtype, const AttnArgs &a, hipStream_t s);
// query rows per prefill row block: the prefill kernel (INT8 and FP8 pools, bf16 queries)
// takes 128, the split kernel's prefill instance kPrefillRows
inline int prefill_block_rows(int format, int q_dtype) { return (format <= 1 && q_dtype == 1) ? 128 : kPrefillRows; }

}  // namespace kvq

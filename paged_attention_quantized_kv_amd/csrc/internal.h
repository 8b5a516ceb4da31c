// internal.h -- shared declarations of the HIP library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvq {

#ifndef KVQ_NT_LOADS
#define KVQ_NT_LOADS 1
#endif
#ifndef KVQ_TEAMS
#define KVQ_TEAMS 2
#endif

constexpr int kPage = 64;                   // token slots per page
constexpr int kTeams = KVQ_TEAMS;           // 4-wave teams per attention workgroup
constexpr int kTargetWgs = 512 / KVQ_TEAMS; // 8 waves per compute unit of the 256-CU chip
constexpr int kMaxChunkPages = 256;   // pages of one decode attention chunk (block ids staged in LDS)
constexpr int kMaxPrefillChunkPages = 4096;  // the same for prefill (262,144 tokens per chunk)
#ifndef KVQ_PREFILL_NT
#define KVQ_PREFILL_NT 4
#endif
#ifndef KVQ_PREFILL_TEAMS
#define KVQ_PREFILL_TEAMS KVQ_TEAMS
#endif
constexpr int kPrefillNT = KVQ_PREFILL_NT;        // 16-row tiles of a prefill row block
constexpr int kPrefillTeams = KVQ_PREFILL_TEAMS;  // 4-wave teams of a prefill workgroup
constexpr int kPrefillRows = 16 * kPrefillNT;   // query rows (t*G + g) of a prefill row block
constexpr int kBulkAppendRows = 64;   // appends of at least this many rows per sequence go page by page

// Launch arguments of kv_append_quant, validated on the host.
struct AppendArgs {
  const void *k_new, *v_new;
  uint8_t *k_codes, *v_codes;
  void *k_scales, *v_scales;
  const int32_t *block_table;
  const int32_t *start_pos;
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
};
constexpr int kMaxBalancedSeqs = 32;
// partial slots (and split workgroups) of a balanced call: one per chunk at most, where every
// (sequence, KV head) may round up by one chunk and a chunk holds at most kMaxChunkPages pages
inline long balanced_slots(long num_seqs, long num_kv_heads, long max_seq_len) {
  const long pages = num_seqs * num_kv_heads * ((max_seq_len + kPage - 1) / kPage);
  const long by_cap = (pages + kMaxChunkPages - 1) / kMaxChunkPages;
  return (by_cap > kTargetWgs ? by_cap : kTargetWgs) + num_seqs * num_kv_heads;
}

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

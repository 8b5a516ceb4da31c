// shape.h -- the host-side shape logic of the library: argument checks of the page pool, the
// split of contexts into chunks and the workspace sizes.  Plain C++ (no HIP), so it builds and
// runs on its own, e.g. under the address and undefined-behaviour sanitizers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/kvq.h"

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
// Per-workgroup cost of a prefill chunk beyond its pages (queries in, partials out), in
// pages: measured at 256K, 128 query rows, between 10 chunks (one round) and 32 (three).
constexpr long kPrefillChunkCost = 16;
constexpr long kPrefillChunkSearch = 1024;  // chunk counts tried above the fewest allowed
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

constexpr int32_t kMaxSeqLen = 1 << 30;  // longest supported context (2^24 pages of 64 tokens)
constexpr int kMaxBalancedSeqs = 64;  // one sequence per lane of the planning wave
// partial slots (and split workgroups) of a balanced call: one per chunk at most, where every
// (sequence, KV head) may round up by one chunk and a chunk holds at most kMaxChunkPages pages
inline long balanced_slots(long num_seqs, long num_kv_heads, long max_seq_len) {
  const long pages = num_seqs * num_kv_heads * ((max_seq_len + kPage - 1) / kPage);
  const long by_cap = (pages + kMaxChunkPages - 1) / kMaxChunkPages;
  return (by_cap > kTargetWgs ? by_cap : kTargetWgs) + num_seqs * num_kv_heads;
}

// KVQ_OK or the status of an invalid or unsupported page-pool descriptor.
int check_cache(const kvq_cache_t *c);

// Tokens per chunk of a decode call: a pure function of the shape (see shape.cpp).
int32_t chunk_tokens(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len);

struct AttnShape {
  int32_t group, rows, tokens_per_split, n_splits;
  bool balanced;  // 2..kMaxBalancedSeqs sequences: chunk length set on the device from the lengths
  int32_t slots;  // partial slots (= split workgroups when balanced)
  size_t ml_bytes, o_bytes;
};
// Shape of a decode call (KVQ_OK, or the status that refuses it).
int attn_shape(int32_t num_seqs, int32_t T, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
               int32_t max_seq_len, AttnShape *s);

struct PrefillShape {
  int32_t group, rows, row_blocks, tokens_per_split, n_splits;
  bool direct;
  size_t ml_bytes, o_bytes;
};
// Shape of a prefill call with row blocks of block_rows query rows.
int prefill_shape(int32_t num_seqs, int32_t T, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t max_seq_len, int block_rows, PrefillShape *s);

// Capacity planning (kvq_page_bytes, kvq_capacity_check in kvq.h).
size_t page_bytes(int32_t format, int32_t head_dim);
int capacity_check(const kvq_cache_t *c, int32_t num_seqs, const int32_t *lens, int32_t max_blocks_per_seq,
                   int64_t *deficit);

}  // namespace kvq

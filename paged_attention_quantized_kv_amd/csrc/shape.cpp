// shape.cpp -- host-side shape logic (shape.h): descriptor checks, chunking, workspace sizes.
#include "shape.h"

#include <algorithm>

namespace kvq {

namespace {
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
}  // namespace

int check_cache(const kvq_cache_t *c) {
  if (!c) return KVQ_ERR_INVALID_ARG;
  if (c->format < KVQ_INT8_G64 || c->format > KVQ_BF16_KV) return KVQ_ERR_INVALID_ARG;
  if (c->num_blocks < 1 || c->num_kv_heads < 1 || c->block_size < 1) return KVQ_ERR_INVALID_ARG;
  if (c->block_size != kPage) return KVQ_ERR_UNSUPPORTED;
  if (c->head_dim != 128 && c->head_dim != 256) return KVQ_ERR_UNSUPPORTED;
  const void *p[4] = {c->k_codes, c->v_codes, c->k_scales, c->v_scales};
  const int n = (c->format == KVQ_BF16_KV) ? 2 : 4;  // the BF16 pool has no scales
  for (int i = 0; i < n; ++i)
    if (!p[i] || !aligned16(p[i])) return KVQ_ERR_INVALID_ARG;
  return KVQ_OK;
}

// Chunking of the context: a pure function of the shape.  Each (sequence, KV head) gets
// as many chunks as keep all workgroups within one per compute unit (at least one), and
// the pages are spread evenly over them, rounded to whole rounds of the workgroup's
// teams.  Past one workgroup per compute unit a second chunk costs a second round and a
// merge, and one chunk per (sequence, KV head) is faster even with compute units idle.
int32_t chunk_tokens(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len) {
  const long pages = (static_cast<long>(max_seq_len) + kPage - 1) / kPage;
  const long units = static_cast<long>(num_seqs) * num_kv_heads;
  long n = units >= kTargetWgs ? 1 : kTargetWgs / units;
  // past kMaxChunkPages per chunk: the fewest chunks that fit, of even length
  n = std::max(n, (pages + kMaxChunkPages - 1) / kMaxChunkPages);
  long pps = (pages + n - 1) / n;
  pps = ((pps + kTeams - 1) / kTeams) * kTeams;
  if (pps < kTeams) pps = kTeams;
  if (pps > kMaxChunkPages) pps = kMaxChunkPages;
  return static_cast<int32_t>(pps * kPage);
}

int attn_shape(int32_t num_seqs, int32_t T, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
               int32_t max_seq_len, AttnShape *s) {
  if (num_seqs < 1 || T < 1 || num_q_heads < 1 || num_kv_heads < 1 || max_seq_len < 1) return KVQ_ERR_INVALID_ARG;
  if (head_dim != 128 && head_dim != 256) return KVQ_ERR_UNSUPPORTED;
  if (num_q_heads % num_kv_heads != 0) return KVQ_ERR_UNSUPPORTED;
  if (T > 8 || num_seqs > 1024 || num_kv_heads > 65535 || max_seq_len > kMaxSeqLen) return KVQ_ERR_UNSUPPORTED;
  const int32_t group = num_q_heads / num_kv_heads;
  if (static_cast<long>(T) * group > 32) return KVQ_ERR_UNSUPPORTED;
  // the merge launches one workgroup per 64-dim slice of every output row
  if (static_cast<long>(num_seqs) * T * num_q_heads * (head_dim / 64) > 0x7FFFFFFFL) return KVQ_ERR_UNSUPPORTED;
  if (max_seq_len < T) return KVQ_ERR_INVALID_ARG;
  s->group = group;
  s->rows = T * group;
  s->tokens_per_split = chunk_tokens(num_seqs, num_kv_heads, max_seq_len);
  s->n_splits = static_cast<int32_t>((static_cast<long>(max_seq_len) + s->tokens_per_split - 1) / s->tokens_per_split);
  // balanced chunking can only split something while the (sequence, KV head) pairs number
  // fewer than the workgroup budget; from there on every pair is one chunk, written directly
  s->balanced = num_seqs >= 2 && num_seqs <= kMaxBalancedSeqs &&
                static_cast<long>(num_seqs) * num_kv_heads < kTargetWgs;
  const long slots = s->balanced ? balanced_slots(num_seqs, num_kv_heads, max_seq_len)
                                 : static_cast<long>(num_seqs) * num_kv_heads * s->n_splits;
  if (slots > 0x7FFFFFFFL) return KVQ_ERR_UNSUPPORTED;
  s->slots = static_cast<int32_t>(slots);
  const size_t parts = static_cast<size_t>(slots) * s->rows;
  s->ml_bytes = ((parts * 2 * sizeof(float)) + 255) & ~static_cast<size_t>(255);
  s->o_bytes = parts * head_dim * sizeof(float);
  return KVQ_OK;
}

// Prefill: any number of query rows T*G per KV head, in blocks of block_rows; the
// context of each (sequence, KV head, row block) is cut into n chunks of at most
// kMaxPrefillChunkPages pages.  A prefill workgroup holds its compute unit alone, so the
// workgroups run in rounds of kTargetWgs: n minimizes rounds x (pages per chunk +
// kPrefillChunkCost), the smallest n within 1% of the best.  With one chunk the kernel
// writes the rows itself (no merge, no partials).
int prefill_shape(int32_t num_seqs, int32_t T, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t max_seq_len, int block_rows, PrefillShape *s) {
  if (num_seqs < 1 || T < 1 || num_q_heads < 1 || num_kv_heads < 1 || max_seq_len < 1) return KVQ_ERR_INVALID_ARG;
  if (head_dim != 128 && head_dim != 256) return KVQ_ERR_UNSUPPORTED;
  if (num_q_heads % num_kv_heads != 0) return KVQ_ERR_UNSUPPORTED;
  if (num_seqs > 1024 || num_kv_heads > 65535 || max_seq_len > kMaxSeqLen) return KVQ_ERR_UNSUPPORTED;
  if (max_seq_len < T) return KVQ_ERR_INVALID_ARG;
  const int32_t group = num_q_heads / num_kv_heads;
  const long rows = static_cast<long>(T) * group;
  const long row_blocks = (rows + block_rows - 1) / block_rows;
  if (rows > 0x7FFFFFFFL || row_blocks * num_kv_heads > 65535) return KVQ_ERR_UNSUPPORTED;
  if (static_cast<long>(num_seqs) * T * num_q_heads * (head_dim / 64) > 0x7FFFFFFFL) return KVQ_ERR_UNSUPPORTED;
  const long pages = (static_cast<long>(max_seq_len) + kPage - 1) / kPage;
  const long units = static_cast<long>(num_seqs) * num_kv_heads * row_blocks;
  auto pages_per_chunk = [&](long n) {
    const long p = ((pages + n - 1) / n + kPrefillTeams - 1) / kPrefillTeams * kPrefillTeams;
    return p < kMaxPrefillChunkPages ? p : static_cast<long>(kMaxPrefillChunkPages);
  };
  auto cost = [&](long n) {
    const long p = pages_per_chunk(n), wgs = (pages + p - 1) / p * units;
    return (wgs + kTargetWgs - 1) / kTargetWgs * (p + kPrefillChunkCost);
  };
  const long nmin = (pages + kMaxPrefillChunkPages - 1) / kMaxPrefillChunkPages;
  long best = cost(nmin);
  for (long n = nmin + 1; n <= pages && n <= nmin + kPrefillChunkSearch; ++n) best = std::min(best, cost(n));
  long n = nmin;
  while (cost(n) * 100 > best * 101) ++n;
  const long pps = pages_per_chunk(n);
  s->group = group;
  s->rows = static_cast<int32_t>(rows);
  s->row_blocks = static_cast<int32_t>(row_blocks);
  s->tokens_per_split = static_cast<int32_t>(pps * kPage);
  s->n_splits = static_cast<int32_t>((pages + pps - 1) / pps);
  s->direct = (s->n_splits == 1);
  const size_t parts = s->direct ? 0 : static_cast<size_t>(num_seqs) * num_kv_heads * s->n_splits * s->rows;
  s->ml_bytes = ((parts * 2 * sizeof(float)) + 255) & ~static_cast<size_t>(255);
  if (s->ml_bytes == 0) s->ml_bytes = 256;
  s->o_bytes = parts * head_dim * sizeof(float);
  return KVQ_OK;
}

// Pool bytes of one page (64 slots of one KV head) over the four arrays of the layout.
size_t page_bytes(int32_t format, int32_t head_dim) {
  if (head_dim != 128 && head_dim != 256) return 0;
  const size_t d = static_cast<size_t>(head_dim), n = kPage;
  switch (format) {
    case KVQ_INT8_G64: return n * (2 * d + 2 * 2 * (d / 64));                   // codes, fp16 group-64 scales
    case KVQ_FP8_E4M3_ROW: return n * (2 * d + 2 * 4);                          // codes, fp32 row scales
    case KVQ_RK8V4: return n * (d + d / 2 + 2 * (d / 64) + 2 * (d / 32));       // int8 K, 4-bit V
    case KVQ_RK4V4: return n * (d / 2 + d / 2 + 2 * (d / 64) + 2 * (d / 32));   // 4-bit K and V
    case KVQ_BF16_KV: return n * 2 * 2 * d;                                     // bf16 K and V, no scales
    default: return 0;
  }
}

int capacity_check(const kvq_cache_t *c, int32_t num_seqs, const int32_t *lens, int32_t max_blocks_per_seq,
                   int64_t *deficit) {
  if (!deficit) return KVQ_ERR_INVALID_ARG;
  *deficit = 0;
  const int rc = check_cache(c);
  if (rc) return rc;
  if (num_seqs < 1 || !lens || max_blocks_per_seq < 1) return KVQ_ERR_INVALID_ARG;
  if (num_seqs > (1 << 20)) return KVQ_ERR_UNSUPPORTED;
  long long blocks = 0, widest = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    if (lens[b] < 0) return KVQ_ERR_INVALID_ARG;
    if (lens[b] > kMaxSeqLen) return KVQ_ERR_UNSUPPORTED;
    const long long pg = (static_cast<long long>(lens[b]) + kPage - 1) / kPage;
    blocks += pg;
    if (pg > widest) widest = pg;
  }
  const long long pool_short = blocks > c->num_blocks ? blocks - c->num_blocks : 0;
  const long long table_short = widest > max_blocks_per_seq ? widest - max_blocks_per_seq : 0;
  // in 128 bits (2^20 sequences of 2^24 pages over 2^31 heads exceed 64), saturated
  const __int128 d = static_cast<__int128>(pool_short) * c->num_kv_heads * page_bytes(c->format, c->head_dim) +
                     static_cast<__int128>(table_short) * num_seqs * 4;
  *deficit = d > static_cast<__int128>(INT64_MAX) ? INT64_MAX : static_cast<int64_t>(d);
  return *deficit == 0 ? KVQ_OK : KVQ_ERR_CAPACITY;
}

}  // namespace kvq

extern "C" {
size_t kvq_page_bytes(int32_t format, int32_t head_dim) { return kvq::page_bytes(format, head_dim); }
int kvq_capacity_check(const kvq_cache_t *cache, int32_t num_seqs, const int32_t *context_lens,
                       int32_t max_blocks_per_seq, int64_t *deficit_bytes) {
  return kvq::capacity_check(cache, num_seqs, context_lens, max_blocks_per_seq, deficit_bytes);
}
}

// kvq_api.hip -- the C ABI (include/kvq.h): host-side validation and dispatch.
//
// Validation is pure host code and runs before any HIP call, so every error
// path can be exercised without a GPU.
#include "../../include/kvq.h"

#include <math.h>

#include <algorithm>
#include <mutex>

#include "internal.h"

namespace {

using kvq::AttnShape;
using kvq::PrefillShape;
using kvq::attn_shape;
using kvq::check_cache;
using kvq::prefill_shape;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

enum class Phase { kBoth, kSplit, kMerge };

int attn_call(Phase phase, const kvq_cache_t *cache, const void *q, int32_t q_dtype, int32_t num_seqs, int32_t T,
              int32_t num_q_heads, const int32_t *block_table, int32_t max_blocks_per_seq, const int32_t *seq_lens,
              int32_t max_seq_len, float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
              void *stream, const void *k_new = nullptr, const void *v_new = nullptr) {
  int rc = check_cache(cache);
  if (rc) return rc;
  if ((k_new == nullptr) != (v_new == nullptr)) return KVQ_ERR_INVALID_ARG;
  if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return KVQ_ERR_INVALID_ARG;
  if (q_dtype != KVQ_F32 && q_dtype != KVQ_BF16) return KVQ_ERR_INVALID_ARG;
  if (!q || !aligned16(q) || !out || !aligned16(out) || !workspace || !aligned16(workspace)) return KVQ_ERR_INVALID_ARG;
  if (!block_table || !aligned4(block_table) || !seq_lens || !aligned4(seq_lens)) return KVQ_ERR_INVALID_ARG;
  if (max_blocks_per_seq < 1) return KVQ_ERR_INVALID_ARG;
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return KVQ_ERR_INVALID_ARG;
  AttnShape s;
  rc = attn_shape(num_seqs, T, num_q_heads, cache->num_kv_heads, cache->head_dim, max_seq_len, &s);
  if (rc) return rc;
  if (static_cast<long>(max_seq_len) > static_cast<long>(max_blocks_per_seq) * kvq::kPage) return KVQ_ERR_CAPACITY;
  if (workspace_bytes < s.ml_bytes + s.o_bytes) return KVQ_ERR_WORKSPACE;

  kvq::AttnArgs a;
  a.k_codes = static_cast<const uint8_t *>(cache->k_codes);
  a.v_codes = static_cast<const uint8_t *>(cache->v_codes);
  a.k_scales = cache->k_scales;
  a.v_scales = cache->v_scales;
  a.q = q;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.ws_ml = static_cast<float *>(workspace);
  a.ws_o = reinterpret_cast<float *>(static_cast<char *>(workspace) + s.ml_bytes);
  a.out = out;
  a.k_new = k_new;
  a.v_new = v_new;
  a.num_seqs = num_seqs;
  a.num_blocks = cache->num_blocks;
  a.num_kv_heads = cache->num_kv_heads;
  a.num_q_heads = num_q_heads;
  a.group = s.group;
  a.T = T;
  a.rows = s.rows;
  a.max_blocks = max_blocks_per_seq;
  a.max_seq_len = max_seq_len;
  a.tokens_per_split = s.tokens_per_split;
  a.balanced = s.balanced ? 1 : 0;
  a.n_splits = s.balanced ? s.slots : s.n_splits;
  a.row_blocks = 1;
  // one call with one chunk per (sequence, KV head): the split kernel writes the normalized
  // rows itself and no merge runs (the two phases called apart keep the partials)
  a.direct_out = (phase == Phase::kBoth && !s.balanced && s.n_splits == 1) ? 1 : 0;
  a.direct_single = (phase == Phase::kBoth && s.balanced) ? 1 : 0;
  a.qk_scale_log2 = softmax_scale * 1.4426950408889634f;

  hipStream_t st = static_cast<hipStream_t>(stream);
  // The step's rows are quantized inside the split launch, except where the row kernel
  // launched first is faster: the rotated formats with more than 16 query rows per KV head,
  // whose fused instance runs out of registers (the 4-bit row quantizer beside two row
  // tiles), and split grids of more than two rounds of workgroups, where every round waits
  // on its workgroups' own row quantization before their pages.
  const long split_wgs = s.balanced ? s.slots : static_cast<long>(num_seqs) * cache->num_kv_heads * s.n_splits;
  const bool rotated_wide = (cache->format == KVQ_RK8V4 || cache->format == KVQ_RK4V4) && s.rows > 16;
  if (k_new && (rotated_wide || split_wgs > 2 * kvq::kTargetWgs)) {
    kvq::AppendArgs ap;
    ap.k_new = k_new;
    ap.v_new = v_new;
    ap.k_codes = static_cast<uint8_t *>(cache->k_codes);
    ap.v_codes = static_cast<uint8_t *>(cache->v_codes);
    ap.k_scales = cache->k_scales;
    ap.v_scales = cache->v_scales;
    ap.block_table = block_table;
    ap.start_pos = seq_lens;  // positions seq_lens[b] - T + t
    ap.start_back = T;
    ap.max_len = max_seq_len;
    ap.num_seqs = num_seqs;
    ap.n_new = T;
    ap.num_kv_heads = cache->num_kv_heads;
    ap.max_blocks = max_blocks_per_seq;
    ap.num_blocks = cache->num_blocks;
    if (kvq::launch_append(cache->format, cache->head_dim, q_dtype, ap, st) != hipSuccess) return KVQ_ERR_LAUNCH;
    a.k_new = a.v_new = nullptr;
  }
  if (phase != Phase::kMerge) {
    if (kvq::launch_attn_split(cache->format, cache->head_dim, q_dtype, a, st) != hipSuccess) return KVQ_ERR_LAUNCH;
  }
  if (phase != Phase::kSplit && a.direct_out == 0) {
    if (kvq::launch_attn_merge(cache->head_dim, a, st) != hipSuccess) return KVQ_ERR_LAUNCH;
  }
  return KVQ_OK;
}

// ---- Scratch of paged_decode_attn_noalloc: a fixed device array instead of a caller's
// workspace.  Every GPU the library runs on holds its own copy until the process ends.  In
// host code `scratch` names a host-side stand-in, so its device address is looked up once
// per device (hipGetSymbolAddress, with that device current) and only that address is used.
constexpr size_t kScratchBytes = 16u << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};

// The scratch address on the current device, or null if it cannot be had.
void *scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

size_t paged_decode_attn_noalloc_max_bytes(void) { return kScratchBytes; }

int paged_decode_attn_noalloc(const kvq_cache_t *cache, const void *q, int32_t q_dtype, int32_t num_seqs, int32_t T,
                              int32_t num_q_heads, const int32_t *block_table, int32_t max_blocks_per_seq,
                              const int32_t *seq_lens, int32_t max_seq_len, float softmax_scale, float *out,
                              void *stream) {
  if (cache == nullptr) return KVQ_ERR_INVALID_ARG;
  // shapes whose partials exceed the scratch are refused before anything else
  {
    const size_t need = paged_decode_attn_workspace_bytes(num_seqs, T, num_q_heads, cache->num_kv_heads,
                                                          cache->head_dim, max_seq_len);
    if (need > kScratchBytes) return KVQ_ERR_WORKSPACE;
  }
  void *ws = scratch_ptr();
  if (ws == nullptr) return KVQ_ERR_LAUNCH;
  return attn_call(Phase::kBoth, cache, q, q_dtype, num_seqs, T, num_q_heads, block_table, max_blocks_per_seq,
                   seq_lens, max_seq_len, softmax_scale, out, ws, kScratchBytes, stream);
}


const char *kvq_status_string(int status) {
  switch (status) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_ERR_INVALID_ARG: return "KVQ_ERR_INVALID_ARG: null or misaligned pointer, bad enum or size";
    case KVQ_ERR_UNSUPPORTED: return "KVQ_ERR_UNSUPPORTED: shape outside the supported set";
    case KVQ_ERR_WORKSPACE: return "KVQ_ERR_WORKSPACE: workspace smaller than paged_decode_attn_workspace_bytes()";
    case KVQ_ERR_CAPACITY: return "KVQ_ERR_CAPACITY: context beyond max_blocks_per_seq * 64";
    case KVQ_ERR_LAUNCH: return "KVQ_ERR_LAUNCH: the HIP runtime refused a kernel launch";
    default: return "KVQ_ERR_UNKNOWN";
  }
}

int kv_append_quant(const kvq_cache_t *cache, const void *k_new, const void *v_new, int32_t src_dtype,
                    int32_t num_seqs, int32_t n_new, const int32_t *block_table, int32_t max_blocks_per_seq,
                    const int32_t *start_pos, void *stream) {
  int rc = check_cache(cache);
  if (rc) return rc;
  if (src_dtype != KVQ_F32 && src_dtype != KVQ_BF16) return KVQ_ERR_INVALID_ARG;
  if (num_seqs < 1 || n_new < 0 || max_blocks_per_seq < 1) return KVQ_ERR_INVALID_ARG;
  if (num_seqs > 1024) return KVQ_ERR_UNSUPPORTED;
  if (!block_table || !aligned4(block_table) || !start_pos || !aligned4(start_pos)) return KVQ_ERR_INVALID_ARG;
  if (n_new == 0) return KVQ_OK;
  if (!k_new || !aligned16(k_new) || !v_new || !aligned16(v_new)) return KVQ_ERR_INVALID_ARG;
  if (static_cast<long>(n_new) > static_cast<long>(max_blocks_per_seq) * kvq::kPage) return KVQ_ERR_CAPACITY;
  const long rows = 2L * num_seqs * n_new * cache->num_kv_heads;
  if ((rows + 3) / 4 > 0x7FFFFFFFL) return KVQ_ERR_UNSUPPORTED;
  kvq::AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_codes = static_cast<uint8_t *>(cache->k_codes);
  a.v_codes = static_cast<uint8_t *>(cache->v_codes);
  a.k_scales = cache->k_scales;
  a.v_scales = cache->v_scales;
  a.block_table = block_table;
  a.start_pos = start_pos;
  a.start_back = 0;
  a.max_len = 0;
  a.num_seqs = num_seqs;
  a.n_new = n_new;
  a.num_kv_heads = cache->num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = cache->num_blocks;
  if (kvq::launch_append(cache->format, cache->head_dim, src_dtype, a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return KVQ_ERR_LAUNCH;
  return KVQ_OK;
}

size_t paged_decode_attn_workspace_bytes(int32_t num_seqs, int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t max_seq_len) {
  AttnShape s;
  if (attn_shape(num_seqs, T, num_q_heads, num_kv_heads, head_dim, max_seq_len, &s) != KVQ_OK) return 0;
  return s.ml_bytes + s.o_bytes;
}

int32_t paged_decode_attn_num_splits(int32_t num_seqs, int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t max_seq_len, int32_t *tokens_per_split) {
  AttnShape s;
  if (attn_shape(num_seqs, T, num_q_heads, num_kv_heads, head_dim, max_seq_len, &s) != KVQ_OK) return 0;
  if (tokens_per_split) *tokens_per_split = s.tokens_per_split;
  return s.n_splits;
}

int paged_decode_attn(const kvq_cache_t *cache, const void *q, int32_t q_dtype, int32_t num_seqs, int32_t T,
                      int32_t num_q_heads, const int32_t *block_table, int32_t max_blocks_per_seq,
                      const int32_t *seq_lens, int32_t max_seq_len, float softmax_scale, float *out, void *workspace,
                      size_t workspace_bytes, void *stream) {
  return attn_call(Phase::kBoth, cache, q, q_dtype, num_seqs, T, num_q_heads, block_table, max_blocks_per_seq,
                   seq_lens, max_seq_len, softmax_scale, out, workspace, workspace_bytes, stream);
}

int paged_decode_attn_split(const kvq_cache_t *cache, const void *q, int32_t q_dtype, int32_t num_seqs, int32_t T,
                            int32_t num_q_heads, const int32_t *block_table, int32_t max_blocks_per_seq,
                            const int32_t *seq_lens, int32_t max_seq_len, float softmax_scale, float *out,
                            void *workspace, size_t workspace_bytes, void *stream) {
  return attn_call(Phase::kSplit, cache, q, q_dtype, num_seqs, T, num_q_heads, block_table, max_blocks_per_seq,
                   seq_lens, max_seq_len, softmax_scale, out, workspace, workspace_bytes, stream);
}

int paged_decode_attn_merge(const kvq_cache_t *cache, const void *q, int32_t q_dtype, int32_t num_seqs, int32_t T,
                            int32_t num_q_heads, const int32_t *block_table, int32_t max_blocks_per_seq,
                            const int32_t *seq_lens, int32_t max_seq_len, float softmax_scale, float *out,
                            void *workspace, size_t workspace_bytes, void *stream) {
  return attn_call(Phase::kMerge, cache, q, q_dtype, num_seqs, T, num_q_heads, block_table, max_blocks_per_seq,
                   seq_lens, max_seq_len, softmax_scale, out, workspace, workspace_bytes, stream);
}

int paged_decode_step(const kvq_cache_t *cache, const void *k_new, const void *v_new, const void *q, int32_t dtype,
                      int32_t num_seqs, int32_t T, int32_t num_q_heads, const int32_t *block_table,
                      int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t max_seq_len, float softmax_scale,
                      float *out, void *workspace, size_t workspace_bytes, void *stream) {
  if (!k_new || !v_new) return KVQ_ERR_INVALID_ARG;
  return attn_call(Phase::kBoth, cache, q, dtype, num_seqs, T, num_q_heads, block_table, max_blocks_per_seq, seq_lens,
                   max_seq_len, softmax_scale, out, workspace, workspace_bytes, stream, k_new, v_new);
}

size_t paged_prefill_attn_workspace_bytes(int32_t num_seqs, int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t max_seq_len) {
  // the larger of the two row-block sizes' needs (the kernel depends on the format and
  // the query dtype, which this query does not take)
  size_t n = 0;
  for (int rows : {128, kvq::kPrefillRows}) {
    PrefillShape s;
    if (prefill_shape(num_seqs, T, num_q_heads, num_kv_heads, head_dim, max_seq_len, rows, &s) != KVQ_OK) return 0;
    n = std::max(n, s.ml_bytes + s.o_bytes);
  }
  return n;
}

int paged_prefill_attn(const kvq_cache_t *cache, const void *q, int32_t q_dtype, int32_t num_seqs, int32_t T,
                       int32_t num_q_heads, const int32_t *block_table, int32_t max_blocks_per_seq,
                       const int32_t *seq_lens, int32_t max_seq_len, float softmax_scale, float *out, void *workspace,
                       size_t workspace_bytes, void *stream) {
  int rc = check_cache(cache);
  if (rc) return rc;
  if (q_dtype != KVQ_F32 && q_dtype != KVQ_BF16) return KVQ_ERR_INVALID_ARG;
  if (!q || !aligned16(q) || !out || !aligned16(out) || !workspace || !aligned16(workspace)) return KVQ_ERR_INVALID_ARG;
  if (!block_table || !aligned4(block_table) || !seq_lens || !aligned4(seq_lens)) return KVQ_ERR_INVALID_ARG;
  if (max_blocks_per_seq < 1) return KVQ_ERR_INVALID_ARG;
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return KVQ_ERR_INVALID_ARG;
  PrefillShape s;
  rc = prefill_shape(num_seqs, T, num_q_heads, cache->num_kv_heads, cache->head_dim, max_seq_len,
                     kvq::prefill_block_rows(cache->format, q_dtype), &s);
  if (rc) return rc;
  if (static_cast<long>(max_seq_len) > static_cast<long>(max_blocks_per_seq) * kvq::kPage) return KVQ_ERR_CAPACITY;
  if (workspace_bytes < s.ml_bytes + s.o_bytes) return KVQ_ERR_WORKSPACE;

  kvq::AttnArgs a;
  a.k_codes = static_cast<const uint8_t *>(cache->k_codes);
  a.v_codes = static_cast<const uint8_t *>(cache->v_codes);
  a.k_scales = cache->k_scales;
  a.v_scales = cache->v_scales;
  a.q = q;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.ws_ml = static_cast<float *>(workspace);
  a.ws_o = reinterpret_cast<float *>(static_cast<char *>(workspace) + s.ml_bytes);
  a.out = out;
  a.k_new = nullptr;
  a.v_new = nullptr;
  a.num_seqs = num_seqs;
  a.num_blocks = cache->num_blocks;
  a.num_kv_heads = cache->num_kv_heads;
  a.num_q_heads = num_q_heads;
  a.group = s.group;
  a.T = T;
  a.rows = s.rows;
  a.max_blocks = max_blocks_per_seq;
  a.max_seq_len = max_seq_len;
  a.tokens_per_split = s.tokens_per_split;
  a.n_splits = s.n_splits;
  a.row_blocks = s.row_blocks;
  a.balanced = 0;
  a.direct_single = 0;
  a.direct_out = s.direct ? 1 : 0;
  a.qk_scale_log2 = softmax_scale * 1.4426950408889634f;

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (kvq::launch_attn_prefill(cache->format, cache->head_dim, q_dtype, a, st) != hipSuccess) return KVQ_ERR_LAUNCH;
  if (!s.direct && kvq::launch_attn_merge(cache->head_dim, a, st) != hipSuccess) return KVQ_ERR_LAUNCH;
  return KVQ_OK;
}

int kvq_check_tables(const kvq_cache_t *cache, int32_t num_seqs, int32_t T, const int32_t *block_table,
                     int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t max_seq_len, int32_t *result,
                     void *stream) {
  int rc = check_cache(cache);
  if (rc) return rc;
  if (num_seqs < 1 || T < 1 || max_blocks_per_seq < 1 || max_seq_len < 1) return KVQ_ERR_INVALID_ARG;
  if (max_seq_len > kvq::kMaxSeqLen) return KVQ_ERR_UNSUPPORTED;
  if (!block_table || !aligned4(block_table) || !seq_lens || !aligned4(seq_lens) || !result || !aligned4(result))
    return KVQ_ERR_INVALID_ARG;
  if (static_cast<long>(max_seq_len) > static_cast<long>(max_blocks_per_seq) * kvq::kPage) return KVQ_ERR_CAPACITY;
  kvq::CheckArgs a;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.result = result;
  a.num_seqs = num_seqs;
  a.T = T;
  a.max_blocks = max_blocks_per_seq;
  a.max_seq_len = max_seq_len;
  a.num_blocks = cache->num_blocks;
  if (kvq::launch_check_tables(a, static_cast<hipStream_t>(stream)) != hipSuccess) return KVQ_ERR_LAUNCH;
  return KVQ_OK;
}

}  // extern "C"

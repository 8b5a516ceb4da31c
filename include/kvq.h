/*
 * kvq.h -- C ABI of the quantized paged KV cache for gfx950 (MI355X).
 *
 * Two operations make up one decode step of a full-attention layer:
 *
 *   kv_append_quant    appends new K/V rows to a paged cache and quantizes them
 *                      on the way in: in the engine of the pages, the append op
 *                      (kv_cache_append) is where KV quantization happens, and
 *                      values are quantized straight from their bf16 source
 *                      (NInfer-3090 README, intro and "RotorQuant KV (rk8v4)").
 *   paged_decode_attn  runs decode attention for 1..B sequences with T query
 *                      rows each (T=1 plain decode, T=4 for an MTP3 verify
 *                      round, whose width is the lane count times the draft
 *                      window plus one: NInfer-3090 README, "Decode after the small-T kernels"),
 *                      dequantizing K/V on the fly over one page pool that all
 *                      sequences share, sized once at startup (gzenz/ninfer
 *                      README, "Current limits").
 *
 * KV formats (NInfer-3090 README, "Choosing a KV format", table):
 *   KVQ_INT8_G64      int8 code per element, one fp16 scale per 64 dims per
 *                     token per KV head (33,792 B/token on the 27B = codes +
 *                     2-byte group scales); scale = fp16_rne(absmax / 127),
 *                     code = clamp(rint(x / scale), -127, 127).
 *   KVQ_FP8_E4M3_ROW  OCP FP8 E4M3FN code per element, one fp32 scale per token
 *                     per KV head = absmax / 448; code = E4M3FN_rne_sat(x / scale).
 *   KVQ_RK8V4         RotorQuant (NInfer-3090 README, "RotorQuant KV (rk8v4)";
 *                     26,112 B/token on the 27B): each 64-dim group of a key row
 *                     is rotated by H64/8, the Sylvester-order Hadamard matrix
 *                     (entry (j, i) = (-1)^popcount(i & j)) over 8, and stored as
 *                     KVQ_INT8_G64; the attention rotates the query by the same
 *                     matrix.  The rotation sums run in binary64 and are rounded
 *                     once to fp32 (exact, so bit-reproducible, for bf16 rows
 *                     unless a group's magnitudes span more than 2^39).  Values are
 *                     not rotated: a signed 4-bit code (-7..7, two's complement)
 *                     per element with one fp16 scale per 32 dims:
 *                     scale = fp16_rne(absmax / 7), code = clamp(rint(x / scale), -7, 7).
 *   KVQ_RK4V4         rk8v4's values; keys rotated as in rk8v4, then each rotated
 *                     dimension is a 4-bit index into the 16-level Lloyd-Max
 *                     quantizer of a unit Gaussian (NInfer-3090 README, "Lloyd-Max
 *                     4-bit keys (rk4v4)"; 17,920 B/token on the 27B).  Level i
 *                     carries the fixed INT8 code rint(127 * L_i / L_15): -127 -96
 *                     -75 -58 -44 -31 -18 -6 6 18 31 44 58 75 96 127 (index 0..15),
 *                     so a key dequantizes as code(index) * scale with the
 *                     KVQ_INT8_G64 group scale fp16_rne(absmax / 127) of the rotated
 *                     group; index = the level whose code is nearest to y / scale
 *                     (fp32), ties to the lower level.
 *   KVQ_BF16_KV       the unquantized reference: each K and V element as bfloat16,
 *                     round to nearest even from the source, no scales (65,536
 *                     B/token on the 27B; NInfer-3090 README, "Choosing a KV
 *                     format").  Attention reads the elements as they are.
 *   A group (or row) whose absmax is 0 stores scale 0 and all-zero codes.
 *
 * Conventions for every call:
 *   - Every pointer is caller-owned DEVICE memory (e.g. torch tensors) unless
 *     stated; the library allocates nothing, never synchronizes, keeps no
 *     state between calls and enqueues work only on `stream` (a hipStream_t;
 *     NULL = the null stream).  Calls are thread-safe.
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid call returns a negative KVQ_ERR_* and enqueues nothing.
 *   - Data pointers (codes, scales, q, k_new, v_new, out, workspace) must be
 *     16-byte aligned; int32 tables 4-byte aligned.
 *   - Device-resident table VALUES (block ids, positions, lengths) are not
 *     readable from the host without a sync, so they are preconditions; the
 *     kernels bounds-check them and never access memory outside the arrays:
 *     an append row whose position or block id is out of range is not
 *     written, and an attention row of a sequence whose length or block ids
 *     are out of range is written as NaN.
 *
 * Supported shapes: block_size 64; head_dim 128 or 256; 1 <= T <= 8;
 * num_q_heads a multiple of num_kv_heads with T * (num_q_heads/num_kv_heads)
 * <= 32; 1 <= num_seqs <= 1024 (paged_prefill_attn takes any T, see there);
 * max_seq_len <= 2^30 tokens.  Anything else returns KVQ_ERR_UNSUPPORTED.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARG = -1, /* null / misaligned pointer, negative size, bad enum */
  KVQ_ERR_UNSUPPORTED = -2, /* shape outside the supported set above */
  KVQ_ERR_WORKSPACE = -3,   /* workspace_bytes below paged_decode_attn_workspace_bytes() */
  KVQ_ERR_CAPACITY = -4,    /* max_seq_len (or start+n_new bound) beyond max_blocks_per_seq * 64;
                               kvq_capacity_check states the shortfall in bytes */
  KVQ_ERR_LAUNCH = -5       /* the HIP runtime refused a launch (no device, bad stream, ...) */
};

typedef enum { KVQ_INT8_G64 = 0, KVQ_FP8_E4M3_ROW = 1, KVQ_RK8V4 = 2, KVQ_RK4V4 = 3, KVQ_BF16_KV = 4 } kvq_format_t;
typedef enum { KVQ_F32 = 0, KVQ_BF16 = 1 } kvq_dtype_t;

/*
 * The page pool.  A page is 64 token slots of one KV head in one block; page
 * (blk, h) is page number p = blk * num_kv_heads + h.
 *
 *   k_codes, v_codes   num_blocks * num_kv_heads * 64 * head_dim bytes; page p
 *                      starts at byte p * 64 * head_dim.  int8 (INT8_G64) or
 *                      E4M3FN bytes (FP8_E4M3_ROW).  RK8V4: k_codes as INT8_G64;
 *                      v_codes 64 * head_dim / 2 bytes per page (4-bit codes).
 *                      RK4V4: k_codes and v_codes 64 * head_dim / 2 bytes per page.
 *                      BF16_KV: k_codes and v_codes 64 * head_dim bf16 per page;
 *                      k_scales and v_scales are not used (may be NULL).
 *   k_scales, v_scales INT8_G64: fp16, 64 * head_dim/64 per page, page p at
 *                      element p * head_dim;  FP8_E4M3_ROW: fp32, 64 per page,
 *                      page p at element p * 64.  RK8V4, RK4V4: k_scales as INT8_G64;
 *                      v_scales fp16, 64 * head_dim/32 per page (element p * 2 * head_dim).
 *
 * Inside a page (s = token slot 0..63, d = dim, D = head_dim, G64 = D/64,
 * run(s) = (s % 16) / 4, pos(s) = (s / 16) * 4 + s % 4):
 *   K byte  ((s/16) * (D/16) + d/16) * 256 + (s%16) * 16 + d%16
 *           (16x16-byte tiles of 16 slots x 16 dims, slot-major inside a tile)
 *   V byte  ((d/16) * 4 + run(s)) * 256 + (d%16) * 16 + pos(s)
 *           (dim-major: the 64 slots of one dim in four 16-byte runs)
 *   INT8 K scale of (s, group g)  element ((run(s) * 4 + s/16) * G64 + g) * 4 + s%4
 *   INT8 V scale of (s, group g)  element (run(s) * G64 + g) * 16 + pos(s)
 *   FP8 K or V scale of s         element run(s) * 16 + pos(s)
 *   RK8V4 K bytes and K scales    as INT8_G64
 *   RK8V4 V code of (s, d)        4 bits at bit 16*(q%2) + 4*(q/2) of the little-endian
 *           32-bit word at byte ((d/32)*64 + run(s)*16 + d%16) * 16 + ((d/16)%2) * 8
 *           + (s/32) * 4, with q = 4 * ((s/16) % 2) + s % 4 (a word holds 8 slots of
 *           one dim; the two 16-dim tiles of a 32-dim pair sit side by side)
 *   RK8V4 V scale of (s, 32-dim group g)  element (run(s) * (D/32) + g) * 16 + pos(s)
 *   RK4V4 V codes and scales, K scales     as RK8V4
 *   BF16_KV K or V element (s, d)  the INT8 K or V byte offset above, in bf16 elements
 *   RK4V4 K index of (s, d)  4 bits at bit 8*(d%4) + 4*((d%8)/4) of the little-endian
 *           32-bit word at byte u * 16 + ((d/64)%2) * 8 + ((d%16)/8) * 4, with
 *           u = ((s/16) * (D/128) + d/128) * 64 + ((d%64)/16) * 16 + s%16
 * These orders make every 64-lane load of the attention kernel one contiguous
 * 1 KiB segment that lands directly in matrix-core operand registers.
 */
typedef struct {
  int32_t format;       /* kvq_format_t */
  int32_t num_blocks;   /* blocks in the pool, >= 1 */
  int32_t block_size;   /* token slots per page: must be 64 */
  int32_t num_kv_heads; /* >= 1 */
  int32_t head_dim;     /* 128 or 256 */
  int32_t reserved;     /* set to 0 */
  void *k_codes;
  void *v_codes;
  void *k_scales;
  void *v_scales;
} kvq_cache_t;

/*
 * kv_append_quant -- quantize n_new rows per sequence and write them into the
 * pool; quantization happens here (NInfer-3090 README, intro).
 *
 *   k_new, v_new        [num_seqs][n_new][num_kv_heads][head_dim] in src_dtype
 *                       (KVQ_BF16 or KVQ_F32); bf16 widens to fp32 exactly.
 *   block_table         [num_seqs][max_blocks_per_seq] int32 block ids.
 *   start_pos           [num_seqs] int32 (device): row t of sequence b goes to
 *                       position start_pos[b] + t, i.e. slot (pos % 64) of block
 *                       block_table[b][pos / 64].
 * Rows of one call must not target the same slot twice.  n_new == 0 is a no-op.
 * Returns KVQ_OK or KVQ_ERR_*; KVQ_ERR_CAPACITY if n_new > max_blocks_per_seq*64.
 */
int kv_append_quant(const kvq_cache_t *cache, const void *k_new, const void *v_new, int32_t src_dtype,
                    int32_t num_seqs, int32_t n_new, const int32_t *block_table,
                    int32_t max_blocks_per_seq, const int32_t *start_pos, void *stream);

/*
 * Bytes of device workspace paged_decode_attn needs for this shape (0 if the
 * shape is unsupported).  The split of each sequence's context into chunks is
 * a pure function of these arguments.
 */
size_t paged_decode_attn_workspace_bytes(int32_t num_seqs, int32_t T, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len);

/*
 * paged_decode_attn -- out = softmax(q k^T * softmax_scale) v over the
 * dequantized cache; every decode step reads the whole cache again, which
 * is why the KV format sets the cost at depth (NInfer-3090 README, "Choosing
 * a KV format").
 *
 *   q          [num_seqs][T][num_q_heads][head_dim] in q_dtype (KVQ_BF16 | KVQ_F32)
 *   seq_lens   [num_seqs] int32 (device): keys visible to the LAST query row of
 *              each sequence, the T new rows included; row t of sequence b sees
 *              keys 0 .. seq_lens[b] - T + t (the T rows are causal among
 *              themselves).  Must satisfy T <= seq_lens[b] <= max_seq_len.
 *   max_seq_len host-side upper bound of seq_lens; sizes the launch grid.
 *   query head h reads KV head h / (num_q_heads / num_kv_heads).
 *   out        [num_seqs][T][num_q_heads][head_dim] fp32.
 *   workspace  >= paged_decode_attn_workspace_bytes(...) bytes, no
 *              initialization needed; calls that share a workspace must be
 *              ordered on one stream.
 * The context of each (sequence, KV head) is cut into chunks attended in
 * parallel and merged with log-sum-exp weights.  2..64 sequences with fewer than
 * 256 (sequence, KV head) pairs: the chunk length is set on the device from the
 * actual lengths, the smallest even number of pages for which all chunks fit one
 * workgroup per compute unit, so short sequences take few chunks and long ones
 * many (num_splits is then only the host's bound).  Otherwise the chunks are those
 * of paged_decode_attn_num_splits(), and when that is one chunk per (sequence, KV
 * head) the chunks write their normalized rows and no merge runs.
 * Accuracy: K/V codes enter the matrix cores exactly (converted to f16); each
 * query row enters scaled by a power of two that puts its largest element in
 * [2^14, 2^15) (its scores take the power of two back), so a bf16 row whose
 * elements lie within 2^28 of its largest is exact in f16 at any magnitude (an
 * fp32 row enters as an f16 hi+lo pair); each
 * softmax weight times its V scale enters as an f16 hi+lo pair, kept inside
 * f16's normal range by two powers of two (one folded into the weights and the
 * row sums, one per wave set from the largest V scale it has seen and taken out
 * of the accumulators at the end), so weights far below the row maximum, e.g.
 * thousands of near-uniform keys under an attention sink, keep their share of
 * the output; all sums are fp32.  Against an fp64 evaluation of the same
 * formula the error is a few 1e-5 at unit-scale inputs and stays below 1e-4 on
 * sink-shaped softmaxes up to 262,144 keys per chunk.
 */
int paged_decode_attn(const kvq_cache_t *cache, const void *q, int32_t q_dtype, int32_t num_seqs,
                      int32_t T, int32_t num_q_heads, const int32_t *block_table,
                      int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t max_seq_len,
                      float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                      void *stream);

/*
 * The same call in its two phases (same arguments, same validation):
 *   _split  each workgroup attends over one chunk of one (sequence, KV head)
 *           and leaves (running max, running sum, unnormalized output) in the
 *           workspace;
 *   _merge  combines the chunks of every query row with log-sum-exp weights
 *           and writes out.
 * paged_decode_attn == _split then _merge on the same stream.
 */
int paged_decode_attn_split(const kvq_cache_t *cache, const void *q, int32_t q_dtype, int32_t num_seqs,
                            int32_t T, int32_t num_q_heads, const int32_t *block_table,
                            int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t max_seq_len,
                            float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                            void *stream);
int paged_decode_attn_merge(const kvq_cache_t *cache, const void *q, int32_t q_dtype, int32_t num_seqs,
                            int32_t T, int32_t num_q_heads, const int32_t *block_table,
                            int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t max_seq_len,
                            float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * paged_decode_step -- one decode step of a full-attention layer in one call:
 * kv_append_quant of the T new rows of every sequence at positions
 * seq_lens[b]-T .. seq_lens[b]-1 (start_pos = seq_lens - T), then
 * paged_decode_attn over the cache including them.  Same results as the two
 * calls in sequence; the rows are quantized inside the attention launch by the
 * workgroup whose context chunk holds them, which saves one launch per step.
 * (Two cases append through a separate launch first, on the same stream, where
 * that is the faster of the two: the rotated formats with more than 16 query rows
 * per KV head, whose fused kernel runs out of registers, and calls of more than
 * 512 attention workgroups, where every round of workgroups would wait on its own
 * rows.)  A sequence whose length is outside [T, max_seq_len] gets no new rows and
 * NaN output rows.
 *
 *   k_new, v_new  [num_seqs][T][num_kv_heads][head_dim], same dtype as q (dtype)
 *   other arguments as for paged_decode_attn (workspace size included).
 */
int paged_decode_step(const kvq_cache_t *cache, const void *k_new, const void *v_new, const void *q, int32_t dtype,
                      int32_t num_seqs, int32_t T, int32_t num_q_heads, const int32_t *block_table,
                      int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t max_seq_len, float softmax_scale,
                      float *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * paged_decode_attn_noalloc -- paged_decode_attn for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, whose place takes a fixed device
 * array inside the library (paged_decode_attn_noalloc_max_bytes() bytes, 16 MiB; each GPU
 * the library runs on holds its own copy until the process ends).  Nothing is allocated.
 * Same kernels and results as paged_decode_attn.  Returns KVQ_ERR_WORKSPACE when the
 * shape's workspace (paged_decode_attn_workspace_bytes) exceeds the array, e.g. 128K-token
 * T=4 calls of one sequence with 24 query / 4 KV heads need ~6.3 MB; KVQ_ERR_LAUNCH if the
 * array's device address cannot be obtained.  All calls on one GPU share the array: calls
 * that may overlap on one GPU (different streams, threads without ordering) race and must
 * not be issued; calls ordered on one stream are safe.
 */
int paged_decode_attn_noalloc(const kvq_cache_t *cache, const void *q, int32_t q_dtype, int32_t num_seqs,
                              int32_t T, int32_t num_q_heads, const int32_t *block_table,
                              int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t max_seq_len,
                              float softmax_scale, float *out, void *stream);
size_t paged_decode_attn_noalloc_max_bytes(void);

/*
 * paged_prefill_attn -- the same attention for a prefill chunk: T query rows per sequence
 * with any T (1 <= T <= max_seq_len; T * (num_q_heads / num_kv_heads) rows per KV head),
 * causal among themselves exactly as in paged_decode_attn (row t sees keys 0 ..
 * seq_lens[b] - T + t).  The chunk's own K/V rows are appended first with
 * kv_append_quant.  This is the step that follows a prefill chunk's append in an
 * engine that prefills in chunks (NInfer-4090 README, "What this fork changes" and
 * "Known limits": chunked prefill attention over the same cache).
 * Arguments as for paged_decode_attn; the workspace is
 * paged_prefill_attn_workspace_bytes() bytes (never 0 for a supported shape).  Rows are
 * handled in blocks of 64 (query row r = t * G + g of a KV head); each (sequence, KV
 * head, row block) streams its context once.  When one chunk per row block fills the
 * chip, the rows are written directly and no merge runs.
 * Supported: head_dim 128 or 256; num_seqs <= 1024; 64-row blocks * num_kv_heads <= 65535.
 * A row's keys are read chunk by chunk up to its last visible key; a block id out of
 * range among the pages of a row's chunks (or a bad seq_lens value) makes the row NaN.
 */
size_t paged_prefill_attn_workspace_bytes(int32_t num_seqs, int32_t T, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len);
int paged_prefill_attn(const kvq_cache_t *cache, const void *q, int32_t q_dtype, int32_t num_seqs,
                       int32_t T, int32_t num_q_heads, const int32_t *block_table,
                       int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t max_seq_len,
                       float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * kvq_check_tables -- debug checker of the device-resident tables that the calls above
 * take as preconditions (the pages require no particular checker; this one exists
 * because block ids and lengths live on the device, where the host cannot read them
 * without a synchronization).  Counts, on `stream`:
 *   result[0]  sequences whose length is outside [T, max_seq_len];
 *   result[1]  block-table entries, among the pages each sequence's length uses
 *              (length clamped to [0, max_seq_len]), outside [0, cache->num_blocks).
 *   result     [2] int32, device memory, overwritten (no initialization needed).
 * Costs one small launch; meant for debugging and tests, not for the decode loop.
 */
int kvq_check_tables(const kvq_cache_t *cache, int32_t num_seqs, int32_t T, const int32_t *block_table,
                     int32_t max_blocks_per_seq, const int32_t *seq_lens, int32_t max_seq_len, int32_t *result,
                     void *stream);

/* Human-readable name of a status code (static string, never NULL). */
const char *kvq_status_string(int status);

/* Number of context chunks per (sequence, KV head) the attention splits a
 * max_seq_len context into, and the tokens per chunk (a multiple of 64);
 * returns 0 for an unsupported shape. */
int32_t paged_decode_attn_num_splits(int32_t num_seqs, int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t max_seq_len, int32_t *tokens_per_split);

/*
 * Capacity planning, host only (nothing is enqueued).  The engine the pages describe
 * refuses a context that does not fit its pool at startup, stating the shortfall to
 * the byte (NInfer-4090 README, "The tradeoff").  Here the caller owns the pool and
 * the block table, so the check takes the planned context lengths and reports what
 * is missing from either.
 *
 * kvq_page_bytes: the pool bytes one page (64 token slots of one KV head) takes in
 * `format` at head_dim, over the four arrays of kvq_cache_t (codes and scales, in the
 * layout above); 0 for an unsupported format or head_dim.
 *
 * kvq_capacity_check: context_lens [num_seqs] int32 in HOST memory, the lengths each
 * sequence will reach.  Sequence b needs ceil(context_lens[b] / 64) blocks, each
 * holding one page per KV head.  *deficit_bytes (host, always written) receives
 *   max(0, sum of blocks - cache->num_blocks) * num_kv_heads * kvq_page_bytes
 *     (pool bytes missing)
 * + max(0, max_b blocks_b - max_blocks_per_seq) * num_seqs * 4
 *     (block-table bytes missing: the [num_seqs][max_blocks_per_seq] int32 table must widen),
 * saturated at INT64_MAX.
 * Returns KVQ_OK when it is 0, KVQ_ERR_CAPACITY otherwise; KVQ_ERR_INVALID_ARG for a bad
 * descriptor, a negative length or null pointers; KVQ_ERR_UNSUPPORTED for a length
 * beyond 2^30 or more than 2^20 sequences.
 */
size_t kvq_page_bytes(int32_t format, int32_t head_dim);
int kvq_capacity_check(const kvq_cache_t *cache, int32_t num_seqs, const int32_t *context_lens,
                       int32_t max_blocks_per_seq, int64_t *deficit_bytes);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */

/*
 * xattn.h -- C ABI of the MI355X (gfx950) XAttention block-sparse
 * chunked-prefill library (libxattn.so).
 *
 * The path has three parts plus a mask reducer and the density counts:
 *   1. xattn_estimate          -- stride-S antidiagonal importance estimate and
 *                                 cumulative-threshold block selection;
 *   2. bsa_prefill             -- block-sparse flash attention over the kept
 *      (bsa_pack_v,              128-token blocks, returning out and LSE
 *       bsa_prefill_packed)      (variant reading V packed once per chunk);
 *   3. attn_merge              -- LSE merge of two partial attention results;
 *   4. xattn_mask_to_cache_blocks -- 128-token block mask -> cache blocks;
 *   5. xattn_density_counts    -- compute / comm density as integer counts.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *     tensors) unless a comment says otherwise.  The caller owns every buffer.
 *     The library never allocates device memory, never frees caller memory
 *     and never synchronises: every call only enqueues kernels on `stream`
 *     (0 = the null stream) and returns.
 *   - Token-major layouts as in the pages' varlen tensors: Q is
 *     [q_len][num_q_heads][head_dim], K and V are [kv_len][num_kv_heads][head_dim],
 *     addressed through element strides (token stride, head stride); the
 *     head_dim axis must be contiguous.  Outputs are dense (layouts below).
 *   - GQA: query head h reads key/value head h / (num_q_heads / num_kv_heads).
 *   - Arguments are validated before anything is launched.  On a non-OK
 *     status nothing has been enqueued and no output was written;
 *     xattn_last_error() returns a thread-local message.  XA_EHIP means a
 *     launch failed (hipGetLastError); outputs are then undefined.
 *   - Batch = 1 per call (one sequence), as the policy on the pages does.
 *   - Thread-safe: no global mutable state besides the thread-local message
 *     and the thread-local measurement events (xattn_set_attention_events).
 */
#ifndef XATTN_H_
#define XATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* xa_stream_t; /* a hipStream_t */
typedef struct ihipEvent_t* xa_event_t;   /* a hipEvent_t */

typedef enum {
  XA_OK = 0,
  XA_EINVAL = 1,        /* bad pointer, size, stride or combination */
  XA_EUNSUPPORTED = 2,  /* valid request outside what the kernels implement */
  XA_EWORKSPACE = 3,    /* workspace missing or smaller than the size query */
  XA_EHIP = 4           /* a HIP launch failed */
} xa_status_t;

typedef enum { XA_F32 = 0, XA_BF16 = 1 } xa_dtype_t;

/* Thread-local text for the last non-OK status returned on this thread. */
const char* xattn_last_error(void);

/* Library version string (static storage). */
const char* xattn_version(void);

/* Measurement hook, not a step of the method.  While set, every call that
 * launches a ping-pong attention kernel (the head-pair or the single-head
 * form; bf16 inputs with head_dim 128
 * through bsa_prefill, bsa_prefill_packed, bsa_prefill_segments,
 * bsa_prefill_varlen or bsa_history_offloaded; fp32 inputs and other head
 * dims run another kernel and record nothing) records `before` on its stream
 * immediately before that launch and `after` immediately after it, so
 * hipEventElapsedTime gives
 * the attention kernel alone, without the work-order kernels and the merge of
 * split halves the call also enqueues.  A call with several such launches
 * (bsa_history_offloaded, one per ring group) leaves the last one in the
 * events.  Both NULL switches the hook off; exactly one NULL is XA_EINVAL.
 * The events are the caller's (hipEventCreate'd, valid while set); the
 * setting belongs to the calling host thread.  A failed record makes the
 * attention call return XA_EHIP. */
xa_status_t xattn_set_attention_events(xa_event_t before, xa_event_t after);

/* ------------------------------------------------------------------------
 * Part 1: importance estimate + block selection  (xattn_estimate_chunked)
 *
 * Follows the XAttention algorithm guide (nano-vllm docs): "Stride Reshape
 * 详解 / Inverse 模式", "Triton Kernels 详解" (flat_group_gemm_fuse_reshape,
 * softmax_fuse_block_sum) and "块选择算法 (find_blocks_chunked)", with the
 * chunk placement of XAttentionBSAPolicy.select_blocks (nano-vllm
 * xattn_bsa.py page).  For query chunk Q (global positions
 * q_start_pos .. q_start_pos+q_len-1) against K rows 0 .. k_len-1
 * (k_len == q_start_pos + q_len):
 *   reshaped row r   = concat_t Q[r*S + S-1-t],  t = 0..S-1
 *   reshaped column c = concat_t K[c*S + t]
 *   z[r][c] = <row r, column c> / (S * sqrt(head_dim)), visible iff
 *             c <= q_start_pos/S + r
 *   P = row softmax over the visible columns
 *   block_scores[h][qb][kb] = sum of P over the (block/S x block/S) tile
 *   block_mask[h][qb][kb] = 1 for kb == 0 and kb == q_start_pos/block + qb
 *     (always kept); the other kb <= that diagonal are ranked by score
 *     (descending, ties by ascending kb) and kept while
 *     (mass of the always-kept blocks + mass ranked before) < threshold * row
 *     total; threshold >= 1 keeps every kb <= diagonal; kb > diagonal = 0.
 *
 * dtype: XA_BF16 (MFMA bf16 x bf16 -> fp32) or XA_F32 (each fp32 value is
 *   split into bf16 hi + lo and three MFMA products are accumulated,
 *   about 16 mantissa bits).
 * Requirements: head_dim in {64, 128}; stride in {2, 4, 8, 16}; block == 128;
 *   q_len, q_start_pos multiples of block; q_len > 0; k_len == q_start_pos + q_len;
 *   k_len / block <= 8192; num_q_heads % num_kv_heads == 0.
 * Outputs (dense, caller-allocated):
 *   block_scores : float   [num_q_heads][q_len/block][k_len/block]
 *   block_mask   : uint8_t [num_q_heads][q_len/block][k_len/block]
 * Workspace: at least xattn_estimate_workspace_size(...) bytes of device
 *   memory, 256-byte aligned; contents on entry are ignored.
 * ------------------------------------------------------------------------ */
size_t xattn_estimate_workspace_size(int64_t q_len, int64_t k_len, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t stride,
                                     int32_t block, xa_dtype_t dtype);

xa_status_t xattn_estimate(const void* q, int64_t q_tok_stride, int64_t q_head_stride,
                           const void* k, int64_t k_tok_stride, int64_t k_head_stride,
                           xa_dtype_t dtype, int64_t q_len, int64_t k_len,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int64_t q_start_pos, int32_t stride, int32_t block, float threshold,
                           float* block_scores, uint8_t* block_mask,
                           void* workspace, size_t workspace_bytes, xa_stream_t stream);

/* ------------------------------------------------------------------------
 * xattn_estimate without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, outputs, kernels and
 * results as xattn_estimate, except that the working memory lives in a
 * device array inside the library (xattn_estimate_noalloc_max_bytes() bytes,
 * 64 MiB: enough for 32 query heads against 131072 keys at stride 8 with
 * bf16 inputs), one copy per GPU, held until the process ends.  The call
 * allocates and frees nothing.  Requirements as for xattn_estimate, plus:
 * the working memory xattn_estimate_workspace_size(...) would ask for must
 * not exceed that maximum (else XA_EUNSUPPORTED, nothing launched), and
 * `stream` must belong to the current device (else XA_EINVAL).  The array
 * needs no clearing between calls; calls that overlap on one GPU (several
 * streams or host threads at once) share it and race: order them.
 * ------------------------------------------------------------------------ */
size_t xattn_estimate_noalloc_max_bytes(void);

xa_status_t xattn_estimate_noalloc(const void* q, int64_t q_tok_stride, int64_t q_head_stride,
                                   const void* k, int64_t k_tok_stride, int64_t k_head_stride,
                                   xa_dtype_t dtype, int64_t q_len, int64_t k_len,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int64_t q_start_pos, int32_t stride, int32_t block, float threshold,
                                   float* block_scores, uint8_t* block_mask, xa_stream_t stream);

/* ------------------------------------------------------------------------
 * Part 2: block-sparse flash attention with LSE  (block_sparse_attn_func /
 * flash_attn_with_lse on the pages)
 *
 * XAttention algorithm guide, "BSA (Block Sparse Attention)"; the history /
 * current-chunk split of XAttentionBSAPolicy.compute_chunked_prefill.
 * K/V row j is global position kv_start + j.  Query row i (global
 * q_start_pos + i) attends to key j iff
 *   mask[h][i/block][(kv_start+j)/block - mask_kb_offset] != 0
 *   and (causal == 0 or kv_start + j <= q_start_pos + i);
 * with s = softmax_scale (0 => 1/sqrt(head_dim)):
 *   lse[h][i] = ln sum_j exp(s q_i.k_j),  out[i][h] = sum_j exp(s q_i.k_j - lse) v_j.
 * A row with no visible key gets out = 0 and lse = -inf.
 * Mask addressing: byte at block_mask + h*mask_head_stride + qb*mask_row_stride + col;
 *   strides may be 0 to broadcast one row to every head / query block;
 *   block_mask == NULL keeps every block (dense).
 * dtype: XA_BF16 (bf16 MFMA, fp32 softmax) or XA_F32 (split bf16 hi/lo, see above).
 * Requirements: head_dim in {64, 128}; block == 128; q_len, q_start_pos,
 *   kv_start multiples of block; kv_len > 0 (any length: the last block may be
 *   partial); num_q_heads % num_kv_heads == 0.
 * Outputs: out  : out_dtype [q_len][num_q_heads][head_dim] (XA_F32 or XA_BF16)
 *          lse  : float [num_q_heads][q_len], natural log.
 * Workspace: at least bsa_prefill_workspace_size(...) bytes (holds V packed as
 *   described under bsa_pack_v, and for XA_F32 the bf16 hi/lo planes of Q and K).
 * ------------------------------------------------------------------------ */
size_t bsa_prefill_workspace_size(int64_t q_len, int64_t kv_len, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, xa_dtype_t dtype);

xa_status_t bsa_prefill(const void* q, int64_t q_tok_stride, int64_t q_head_stride,
                        const void* k, int64_t k_tok_stride, int64_t k_head_stride,
                        const void* v, int64_t v_tok_stride, int64_t v_head_stride,
                        xa_dtype_t dtype, int64_t q_len, int64_t kv_len,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int64_t q_start_pos, int64_t kv_start,
                        const uint8_t* block_mask, int64_t mask_head_stride,
                        int64_t mask_row_stride, int64_t mask_kb_offset,
                        int32_t block, int32_t causal, float softmax_scale,
                        void* out, xa_dtype_t out_dtype, float* lse,
                        void* workspace, size_t workspace_bytes, xa_stream_t stream);

/* ------------------------------------------------------------------------
 * Packed V for repeated attention calls over one growing key/value cache
 *
 * The attention kernel reads V transposed (per kv head: head_dim rows of
 * tokens, keys permuted inside each group of 16 into the order the MFMA
 * fragments use).  bsa_prefill builds that layout in its workspace on every
 * call; for chunked prefill (XAttentionBSAPolicy.compute_chunked_prefill: each
 * chunk attends the whole history, then its own keys) the caller can instead
 * pack each chunk's V rows once, when they are produced, and call
 * bsa_prefill_packed for every later chunk.
 *
 * bsa_packed_v_bytes: bytes of a packed buffer holding `capacity` tokens
 *   (rounded up to 128) for num_kv_heads heads (two bf16 planes for XA_F32).
 * bsa_pack_v: writes V rows 0 .. n_tokens-1 ([n_tokens][hkv][head_dim],
 *   strided, dtype XA_BF16 or XA_F32) as packed tokens token_offset ..
 *   token_offset+n_tokens-1; packed tokens up to the next multiple of 128 are
 *   zeroed.  token_offset must be a multiple of 128 and the range must fit in
 *   capacity.  packed_v must be 256-byte aligned device memory.
 * bsa_prefill_packed: bsa_prefill with V taken from packed tokens
 *   v_token_offset .. v_token_offset+kv_len-1 of packed_v (a multiple of 128;
 *   same dtype as when packed).  Workspace: bsa_prefill_packed_workspace_size
 *   bytes (0 for XA_BF16; workspace may then be NULL).
 * ------------------------------------------------------------------------ */
size_t bsa_packed_v_bytes(int64_t capacity, int32_t num_kv_heads, int32_t head_dim, xa_dtype_t dtype);

xa_status_t bsa_pack_v(const void* v, int64_t v_tok_stride, int64_t v_head_stride, xa_dtype_t dtype,
                       int64_t n_tokens, int32_t num_kv_heads, int32_t head_dim, void* packed_v,
                       int64_t capacity, int64_t token_offset, xa_stream_t stream);

size_t bsa_prefill_packed_workspace_size(int64_t q_len, int64_t kv_len, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim, xa_dtype_t dtype);

xa_status_t bsa_prefill_packed(const void* q, int64_t q_tok_stride, int64_t q_head_stride,
                               const void* k, int64_t k_tok_stride, int64_t k_head_stride,
                               const void* packed_v, int64_t capacity, int64_t v_token_offset,
                               xa_dtype_t dtype, int64_t q_len, int64_t kv_len,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int64_t q_start_pos, int64_t kv_start,
                               const uint8_t* block_mask, int64_t mask_head_stride,
                               int64_t mask_row_stride, int64_t mask_kb_offset,
                               int32_t block, int32_t causal, float softmax_scale,
                               void* out, xa_dtype_t out_dtype, float* lse,
                               void* workspace, size_t workspace_bytes, xa_stream_t stream);

/* ------------------------------------------------------------------------
 * Several attention problems over one query chunk in a single launch
 *
 * XAttentionBSAPolicy.compute_chunked_prefill attends a chunk twice -- the
 * history without the causal rule and the chunk's own keys with it -- and
 * merges the two partials.  bsa_prefill_segments runs up to 4 such segments
 * (each exactly a bsa_prefill_packed call with its own keys, packed-V range,
 * mask, causal flag and outputs, sharing Q, heads and the packed-V buffer) as
 * one grid.  segments: HOST array of n_segments (1..4) descriptors.  XA_BF16
 * inputs only.
 *
 * Work order: each (segment, query head, query block) row of kept key blocks
 * is one work item.  Two small kernels on the same stream count every item's
 * kept blocks, split each item longer than the mean load per resident
 * workgroup (up to 512 items) into two halves at its median kept block, and
 * sort the entries longest first; the attention workgroups take entries in
 * that order as they start, so no long row trails at the end of the grid, and
 * a last kernel merges each split item's halves by their LSE (as attn_merge
 * does).  The order decides only which workgroup computes what: results equal
 * those of the unsplit computation up to fp32 rounding.
 * workspace: at least bsa_prefill_segments_workspace_size(q_len, num_q_heads,
 * head_dim, n_segments) bytes of 256-byte aligned device memory (the order
 * plus fp32 partial results of up to 512 split items: 64.5 MiB at head_dim
 * 128 once there are 512 or more items), owned by the caller and used only by
 * this call while it runs (two calls in flight at once need two workspaces);
 * contents need no initialisation.  XA_EWORKSPACE if missing or too small.
 * Validation of every segment precedes the launch; other errors as for
 * bsa_prefill_packed.
 * ------------------------------------------------------------------------ */
typedef struct {
  const void* k;               /* [kv_len][num_kv_heads][head_dim] key rows of this segment */
  int64_t k_tok_stride, k_head_stride;
  int64_t kv_len, kv_start;    /* key row j is global position kv_start + j */
  int64_t v_token_offset;      /* packed-V tokens v_token_offset .. +kv_len hold V of these rows */
  const uint8_t* block_mask;   /* as for bsa_prefill; NULL = every block */
  int64_t mask_head_stride, mask_row_stride, mask_kb_offset;
  int32_t causal;
  void* out;                   /* out_dtype [q_len][num_q_heads][head_dim] */
  float* lse;                  /* [num_q_heads][q_len] */
} xa_segment_t;

/* Bytes of the work-order workspace for items = n_segments * num_q_heads *
 * ceil(q_len / 128) work items; 0 for invalid sizes. */
size_t bsa_prefill_segments_workspace_size(int64_t q_len, int32_t num_q_heads, int32_t head_dim,
                                           int32_t n_segments);

xa_status_t bsa_prefill_segments(const void* q, int64_t q_tok_stride, int64_t q_head_stride,
                                 const void* packed_v, int64_t capacity, xa_dtype_t dtype,
                                 int64_t q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int64_t q_start_pos,
                                 const xa_segment_t* segments, int32_t n_segments,
                                 int32_t block, float softmax_scale, xa_dtype_t out_dtype,
                                 void* workspace, size_t workspace_bytes, xa_stream_t stream);

/* ------------------------------------------------------------------------
 * Estimate against downsampled history keys (metadata of offloaded K)
 *
 * Task plan page, "Metadata 存储策略" scheme A and "Phase 3: select_blocks
 * 实现": every stride-th key token of each offloaded block is kept on the
 * GPU, and a query chunk is estimated against that downsampled history with
 * stride 1 and blocks of block / stride rows (one block of downsampled keys
 * stands for one 128-token history block).  Per (query token, downsampled
 * key) the logit is q.k / sqrt(head_dim); each row is normalised over all
 * history keys (they all precede the chunk: no causal limit); block scores
 * are the sums over (block/stride x block/stride) tiles; selection per row as
 * xattn_estimate with block 0 the only forced block (the chunk's diagonal
 * block lies past the history).  The union over heads and query blocks, by
 * cache block, is xattn_mask_to_cache_blocks on the returned mask.
 *
 * xattn_downsample_keys: rows ds_offset .. ds_offset + n_tokens/stride - 1 of
 *   k_ds ([ds_capacity][num_kv_heads][head_dim], dense, same dtype) become
 *   key rows 0, stride, 2*stride, ... of k (strided as for xattn_estimate).
 *   n_tokens must be a multiple of stride; k_ds 16-byte aligned.
 * xattn_estimate_history_ds: q [q_len][num_q_heads][head_dim] (strided),
 *   k_ds [n_ds][num_kv_heads][head_dim] (strided); q_len and n_ds multiples
 *   of b = block / stride; block 128, stride in {2, 4, 8, 16}.
 *   block_scores float [num_q_heads][q_len/b][n_ds/b], block_mask uint8 of the
 *   same shape; workspace of xattn_estimate_history_ds_workspace_size bytes
 *   (256-byte aligned): per (head, key block, query token) a log-sum-exp
 *   partial, num_q_heads * (n_ds/b) * q_len floats (plus bf16 hi/lo planes of
 *   Q and K for XA_F32).  Errors as for xattn_estimate.
 * ------------------------------------------------------------------------ */
xa_status_t xattn_downsample_keys(const void* k, int64_t k_tok_stride, int64_t k_head_stride, xa_dtype_t dtype,
                                  int64_t n_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t stride,
                                  void* k_ds, int64_t ds_capacity, int64_t ds_offset, xa_stream_t stream);

size_t xattn_estimate_history_ds_workspace_size(int64_t q_len, int64_t n_ds, int32_t num_q_heads,
                                                int32_t num_kv_heads, int32_t head_dim, int32_t stride,
                                                int32_t block, xa_dtype_t dtype);

xa_status_t xattn_estimate_history_ds(const void* q, int64_t q_tok_stride, int64_t q_head_stride,
                                      const void* k_ds, int64_t k_tok_stride, int64_t k_head_stride,
                                      xa_dtype_t dtype, int64_t q_len, int64_t n_ds,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t stride, int32_t block, float threshold,
                                      float* block_scores, uint8_t* block_mask,
                                      void* workspace, size_t workspace_bytes, xa_stream_t stream);

/* ------------------------------------------------------------------------
 * Offloaded history (cache blocks in pinned host memory)
 *
 * XAttentionBSAPolicy page, compute_chunked_prefill with the offload engine
 * (the history comes from CPU cache blocks through a ring of GPU slots) and
 * task plan page, "核心设计理解" (1 CPU block = 8 BSA blocks).  A host store
 * of n_host_blocks cache blocks of cache_block tokens holds K token-major,
 * host_k [n_host_blocks * cache_block][num_kv_heads][head_dim], and V packed
 * for the attention kernel over the whole store, host_vt [num_kv_heads]
 * [head_dim][n_host_blocks * cache_block] (keys permuted in groups of 16 as
 * bsa_pack_v does); bf16, pinned memory for asynchronous copies, owned by the
 * caller.  Consecutive cache blocks are thus one K copy and one 2-D V copy.
 *
 * xattn_offload_blocks: stores n_blocks consecutive cache blocks of k / v
 *   (device, [n_blocks * cache_block][num_kv_heads][head_dim], head_dim
 *   contiguous and heads contiguous within a token for k) as host blocks
 *   first_block ..; V is packed into staging_vt (device, 256-byte aligned,
 *   n_blocks * num_kv_heads * head_dim * cache_block bf16) first.  Copies are
 *   queued on stream; host memory is written when the stream reaches them.
 * bsa_history_offloaded: attention of the query chunk q ([q_len][num_q_heads]
 *   [head_dim] bf16, strided; global position q_start_pos) over every token of
 *   the host cache blocks keep[0 .. n_keep-1] (HOST array, ids < n_host_blocks)
 *   without the causal rule (history).  The blocks move in groups of `group`
 *   into a device ring of 2 * group blocks -- ring_k [2*group*cache_block]
 *   [num_kv_heads][head_dim] and ring_vt, packed V of capacity 2 * group *
 *   cache_block (256-byte aligned) -- on copy_stream (one K copy and one
 *   2-D V copy per run of consecutive ids), the attention over a
 *   group runs on stream once its copies land (events order the two streams
 *   both ways), and each group's result (part_out / part_lse, same shapes as
 *   out / lse) is merged into out / lse by LSE (attn_merge).  out bf16
 *   [q_len][num_q_heads][head_dim], lse float [num_q_heads][q_len]; n_keep = 0
 *   gives out 0 and lse -inf.  Copies into the ring wait for all work queued on
 *   stream before the call.  Errors as for bsa_prefill_packed.
 * ------------------------------------------------------------------------ */
xa_status_t xattn_offload_blocks(const void* k, int64_t k_tok_stride, int64_t k_head_stride, const void* v,
                                 int64_t v_tok_stride, int64_t v_head_stride, xa_dtype_t dtype, int32_t n_blocks,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t cache_block, void* host_k,
                                 void* host_vt, int64_t n_host_blocks, int64_t first_block, void* staging_vt,
                                 xa_stream_t stream);

xa_status_t bsa_history_offloaded(const void* q, int64_t q_tok_stride, int64_t q_head_stride, xa_dtype_t dtype,
                                  int64_t q_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int64_t q_start_pos, const void* host_k, const void* host_vt,
                                  int64_t n_host_blocks, int32_t cache_block, const int32_t* keep, int32_t n_keep,
                                  int32_t group, void* ring_k, void* ring_vt, void* out, float* lse,
                                  void* part_out, float* part_lse, xa_stream_t stream, xa_stream_t copy_stream);

/* xattn_estimate_offloaded: xattn_estimate (same scores and mask, bit for bit)
 *   of the query chunk q ([q_len][num_q_heads][head_dim] bf16, global position
 *   q_start_pos) against keys 0 .. q_start_pos + q_len - 1 where the history
 *   keys 0 .. q_start_pos - 1 are the host cache blocks 0 .. q_start_pos /
 *   cache_block - 1 of host_k (q_start_pos a multiple of cache_block) and the
 *   chunk's own keys are k_cur ([q_len][num_kv_heads][head_dim] bf16 on the
 *   device).  XAttentionBSAPolicy page, select_blocks: the estimate runs over
 *   the keys as they arrive from the CPU cache, a group of cache blocks at a
 *   time (per-row partial statistics per key chunk, merged before the block
 *   sums).  Every history block passes once through ring_k (the K half of the
 *   ring of bsa_history_offloaded, 2 * group * cache_block tokens): copies on
 *   copy_stream, estimate GEMMs on stream, events both ways; the partial
 *   log-sum-exp of each (row, key block) goes to the workspace and one
 *   selection pass finishes on stream.  Workspace: xattn_estimate_workspace_
 *   size(q_len, q_start_pos + q_len, ..., XA_BF16) bytes, 256-byte aligned.
 *   block_scores / block_mask as for xattn_estimate ([num_q_heads][q_len /
 *   128][(q_start_pos + q_len) / 128]).  Copies into the ring wait for all
 *   work queued on stream before the call.  Errors: XA_EUNSUPPORTED for
 *   other dtypes, head dims, strides or blocks; XA_EINVAL for shapes, null
 *   pointers or alignment; XA_EWORKSPACE for a short workspace; nothing is
 *   queued on an error.
 */
xa_status_t xattn_estimate_offloaded(const void* q, int64_t q_tok_stride, int64_t q_head_stride, const void* k_cur,
                                     int64_t kc_tok_stride, int64_t kc_head_stride, xa_dtype_t dtype, int64_t q_len,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int64_t q_start_pos, const void* host_k, int64_t n_host_blocks,
                                     int32_t cache_block, int32_t group, void* ring_k, int32_t stride,
                                     int32_t block, float threshold, float* block_scores, uint8_t* block_mask,
                                     void* workspace, size_t workspace_bytes, xa_stream_t stream,
                                     xa_stream_t copy_stream);

/* ------------------------------------------------------------------------
 * Packed batch of sequences (varlen)
 *
 * XAttentionBSAPolicy page, compute_prefill (GPU-only mode): Q [total_q][heads][d] and
 * K / V [total_kv][kv_heads][d] packed sequence after sequence, with
 * cumulative lengths cu_seqlens_q / cu_seqlens_k [batch + 1]; the page runs
 * the estimate and the block-sparse attention for one sequence and leaves
 * batches above one to dense attention.  Here sequence b is its own
 * problem: queries rows cu_q[b] .. cu_q[b+1]-1 at global positions
 * k_len_b - q_len_b .. (the queries end where the keys end), keys rows
 * cu_k[b] .. cu_k[b+1]-1, causal; every sequence of the batch runs in one
 * grid per kernel (one estimate GEMM, one selection, one attention with a
 * work order across all sequences).
 *
 * cu_seqlens_q / cu_seqlens_k: HOST arrays of batch + 1 int64, starting at
 * 0, non-decreasing; every q_len_b and k_len_b a multiple of 128 with
 * q_len_b <= k_len_b (a sequence with q_len_b = 0 contributes nothing);
 * 1 <= batch <= 65536; at most 8192 key blocks per sequence.  bf16 inputs,
 * head_dim 128.
 *
 * Scores / mask of a batch: sequence b's [num_q_heads][q_len_b/128]
 * [k_len_b/128] block after those of sequences 0..b-1 (element offset the
 * sum of the earlier blocks; xattn_varlen_mask_elems gives the total, -1 on
 * invalid lengths).  Out: [total_q][num_q_heads][head_dim] rows as q.  LSE:
 * sequence b's [num_q_heads][q_len_b] block at float offset num_q_heads *
 * cu_q[b].
 *
 * xattn_estimate_varlen: xattn_estimate of every sequence (its q_start_pos =
 *   k_len_b - q_len_b), stride in {2, 4, 8, 16}, block 128; workspace of
 *   xattn_estimate_varlen_workspace_size bytes (256-byte aligned): the
 *   sequence records and the per-(row, key block) LSE partials.
 * bsa_prefill_varlen: bsa_prefill of every sequence with its mask block
 *   (block_mask null: dense causal); packed_v holds the batch's V packed by
 *   bsa_pack_v as tokens 0 .. total_kv - 1 (capacity >= total_kv); workspace
 *   of bsa_prefill_varlen_workspace_size bytes (records and work order).
 * Errors as for the single-sequence calls; nothing is queued on an error.
 * ------------------------------------------------------------------------ */
int64_t xattn_varlen_mask_elems(const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_k, int32_t batch,
                                int32_t num_q_heads);
size_t xattn_estimate_varlen_workspace_size(const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_k, int32_t batch,
                                            int32_t num_q_heads, int32_t num_kv_heads, int32_t stride);
xa_status_t xattn_estimate_varlen(const void* q, int64_t q_tok_stride, int64_t q_head_stride, const void* k,
                                  int64_t k_tok_stride, int64_t k_head_stride, xa_dtype_t dtype,
                                  const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_k, int32_t batch,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t stride,
                                  int32_t block, float threshold, float* block_scores, uint8_t* block_mask,
                                  void* workspace, size_t workspace_bytes, xa_stream_t stream);
size_t bsa_prefill_varlen_workspace_size(const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_k, int32_t batch,
                                         int32_t num_q_heads, int32_t head_dim);
xa_status_t bsa_prefill_varlen(const void* q, int64_t q_tok_stride, int64_t q_head_stride, const void* k,
                               int64_t k_tok_stride, int64_t k_head_stride, const void* packed_v, int64_t capacity,
                               xa_dtype_t dtype, const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_k,
                               int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               const uint8_t* block_mask, int32_t block, float softmax_scale, void* out,
                               xa_dtype_t out_dtype, float* lse, void* workspace, size_t workspace_bytes,
                               xa_stream_t stream);

/* ------------------------------------------------------------------------
 * Part 3: LSE merge  (merge_attention_outputs)
 *
 * nano-vllm CLAUDE.md, "Online Softmax Merge - Triton Fused Kernel":
 *   m = max(lse_a, lse_b); e_x = exp(lse_x - m);
 *   lse_out = m + ln(e_a + e_b);  o_out = (o_a e_a + o_b e_b) / (e_a + e_b).
 * Both lse = -inf gives o_out = 0, lse_out = -inf; one -inf returns the other.
 * o_*: o_dtype [q_len][heads][head_dim] dense; lse_*: float [heads][q_len].
 * Math in fp32.  o_out may alias o_a or o_b, lse_out may alias lse_a or lse_b
 * (each element is read before it is written by the same thread).
 * Requirements: q_len >= 0, heads > 0, head_dim > 0 and head_dim % 8 == 0.
 * ------------------------------------------------------------------------ */
xa_status_t attn_merge(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                       void* o_out, float* lse_out, xa_dtype_t o_dtype,
                       int64_t q_len, int32_t heads, int32_t head_dim, xa_stream_t stream);

/* ------------------------------------------------------------------------
 * 128-token block mask -> cache blocks
 *
 * Task plan page (nano-vllm task_plan.md), "select_blocks 设计" step 3, and
 * XAttentionBSAPolicy.select_blocks step 6: a cache block of sub_blocks
 * consecutive 128-token blocks is kept if any of them is selected; the union
 * over heads and query blocks is the list of cache blocks to load, with the
 * first and last history cache block always included (force_first_last).
 *   mask byte (h, qb, col) at block_mask + h*mask_head_stride + qb*mask_row_stride + col
 *   cache block cb covers columns kb_begin + cb*sub_blocks .. (clipped to n_cols)
 * Outputs (each may be NULL):
 *   keep_per_head : uint8_t [heads][n_qb][n_cache_blocks]
 *   keep_any      : uint8_t [n_cache_blocks]
 *   keep_any_blocks : uint8_t [n_cache_blocks * sub_blocks] -- keep_any
 *                     expanded back to 128-token columns (a broadcast mask
 *                     row for bsa_prefill with zero head/row strides).
 * Requirements: heads, n_qb, sub_blocks > 0; 0 <= kb_begin; n_cache_blocks >= 0;
 *   kb_begin + (n_cache_blocks-1)*sub_blocks < n_cols when n_cache_blocks > 0.
 * ------------------------------------------------------------------------ */
xa_status_t xattn_mask_to_cache_blocks(const uint8_t* block_mask, int32_t heads, int32_t n_qb,
                                       int64_t n_cols, int64_t mask_head_stride,
                                       int64_t mask_row_stride, int64_t kb_begin,
                                       int64_t n_cache_blocks, int32_t sub_blocks,
                                       int32_t force_first_last, uint8_t* keep_per_head,
                                       uint8_t* keep_any, uint8_t* keep_any_blocks,
                                       xa_stream_t stream);

/* ------------------------------------------------------------------------
 * Density counts (compute density and comm density)
 *
 * XAttentionBSAPolicy.select_blocks, "Step 5: Record density": the compute
 * density of a chunk is the number of kept (head, query block, key block)
 * pairs on or below the causal diagonal over the number of such pairs; and
 * the comm density recorded after step 6: the cache blocks to load over the
 * cache blocks the history holds.  Integer counts, so a whole prefill's
 * density is one ratio of sums (the policy's statistics accumulate the same
 * way across chunks).
 *   mask byte (h, qb, col) at block_mask + h*mask_head_stride + qb*mask_row_stride + col;
 *   row qb's causal columns are 0 .. min(diag0 + qb, n_cols - 1) (diag0 = the
 *   column of query block 0's diagonal block, q_start_pos/128 for a chunk's
 *   mask whose column 0 is key block 0; diag0 >= n_cols - 1 counts every column,
 *   as for a history-only mask).
 * counts: int64_t[4] in DEVICE memory, 8-byte aligned, ADDED to (the caller
 *   zeroes it):
 *   counts[0] += kept causal pairs        counts[1] += causal pairs
 *   counts[2] += nonzero keep_any bytes   counts[3] += n_cache_blocks
 * block_mask may be NULL (counts[0..1] unchanged; heads, n_qb, n_cols, strides
 *   ignored); keep_any may be NULL when n_cache_blocks == 0 (counts[2..3]
 *   unchanged).  keep_any: uint8_t[n_cache_blocks], e.g. the keep_any output
 *   of xattn_mask_to_cache_blocks.
 * Errors: XA_EINVAL for a null or misaligned counts, heads/n_qb/n_cols <= 0 or
 *   a negative stride with a mask, n_cache_blocks < 0, or n_cache_blocks > 0
 *   without keep_any; nothing is launched then.
 * ------------------------------------------------------------------------ */
xa_status_t xattn_density_counts(const uint8_t* block_mask, int32_t heads, int32_t n_qb, int64_t n_cols,
                                 int64_t mask_head_stride, int64_t mask_row_stride, int64_t diag0,
                                 const uint8_t* keep_any, int64_t n_cache_blocks, int64_t* counts,
                                 xa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* XATTN_H_ */

/*
 * pkv.h -- C ABI of libpkv: attention over a flat, slot-addressed KV pool
 * (one-token pages, or pages of a power-of-two token count) on AMD Instinct
 * MI355X (gfx950).
 *
 * Data model (AstrAI "Inference" guide, section "KVCache System"):
 *   k_buffer, v_buffer   [n_layers, size, n_kv_heads, head_dim], one dtype
 *   req_to_token         int32 [num_reqs, max_ctx_len]: logical position ->
 *                        physical slot of the pool (one-token pages), or,
 *                        for pools of page_size > 1 tokens per page, int32
 *                        [num_reqs, ceil(max_ctx_len / page_size)]: logical
 *                        page -> physical page (see pkv_pool)
 *   per step             req_pool_indices[B], seq_lens[B], kv_indptr[B+1],
 *                        qo_indptr[B+1], out_cache_loc[n_new], host max_len
 * Cached keys are already rotated: RoPE happens before the cache write
 * (same guide, section "KV Cache"), so no kernel here rotates anything.
 * All index arrays are int32 (commit history of tests/inference/test_cache.py,
 * entry on int32 page-table, request-row and cache-location indices).
 *
 * Conventions for every entry point:
 *   - "device" pointers are HIP device memory of the current device; "host"
 *     pointers are ordinary CPU memory.  The caller owns every buffer.
 *   - The library never allocates or frees device memory, never synchronises
 *     the device, and keeps no state between calls except the per-device
 *     address of its one static scratch array (pkv_paged_decode_store_noalloc);
 *     calls are re-entrant and thread-safe, except that calls of that one
 *     entry point which overlap on one device share its scratch and race.
 *   - Kernels are enqueued on the caller's stream and return before they run.
 *   - Host-checkable arguments are validated and reported as a pkv_status;
 *     nothing is launched when a check fails.  Device-resident metadata is
 *     NOT read on the host: inconsistent metadata (out-of-range slots, wrong
 *     prefix sums) is undefined behaviour unless pkv_validate_step accepted
 *     a host copy of it first.
 *   - Offsets into the pool are computed in 64-bit arithmetic.
 *   - Supported: key / value widths (head_dim, v_head_dim) of (64, 64) or
 *     (128, 128), and MLA-shaped (192, 128) in bf16; dtype f32 or bf16
 *     (prefill: bf16 only); n_heads a multiple of n_kv_heads; page_size 1 or
 *     a power of two up to 65536.  Queries are head_dim wide, attention
 *     outputs and decode partials v_head_dim wide.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,                 /* a required pointer is NULL            */
  PKV_ERR_SHAPE = 2,                /* a size / count / layer out of range   */
  PKV_ERR_DTYPE = 3,                /* dtype unsupported for this call       */
  PKV_ERR_WORKSPACE_TOO_SMALL = 4,  /* workspace below the required size     */
  PKV_ERR_BAD_METADATA = 5,         /* pkv_validate_step / pkv_build_step    */
  PKV_ERR_HIP = 6,                  /* a HIP runtime call or launch failed   */
  PKV_ERR_UNSUPPORTED = 7,          /* valid but not implemented (head_dim)  */
  PKV_ERR_SCRATCH_LIMIT = 8         /* needs more than the static scratch    */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;

/* How the bf16 matrix-core decode kernels read K/V rows (pkv_pool.load_policy).
 * The same section's allocator and prefix cache let requests share prompt
 * slots; rows that another request of the step (or the next layer pass)
 * reads again are worth keeping in the caches, rows read once are not.
 *   PKV_LOAD_AUTO    (0) non-temporal row loads for a decode step of one
 *                        request whose K/V over all n_layers of the pool
 *                        exceed the 256 MiB last-level cache (nothing of it
 *                        survives until it is read again); cached loads
 *                        otherwise.  See pkv_decode_load_kind.
 *   PKV_LOAD_CACHED  (1) always cached loads.
 *   PKV_LOAD_STREAM  (2) always non-temporal row loads: for callers whose
 *                        allocator never gives two requests the same slot.
 * Affects speed only: results are the same bits under every policy.  The
 * shared-prefix step, the one-launch step and the vector kernels (fp32,
 * head_dim 64) always use cached loads. */
typedef enum { PKV_LOAD_AUTO = 0, PKV_LOAD_CACHED = 1, PKV_LOAD_STREAM = 2 } pkv_load_policy;

/* KVStorage + ReqToTokenPool ("Inference" guide, section "KVCache System").
 *
 * Pages.  The same section runs the pool in paged mode with page_size 1 or
 * larger; the PagedCache of the v1.3.3 -> v1.3.4 compare page stores its
 * caches as [n_layers, n_pages, page_size, n_kv_heads, head_dim] and puts
 * logical position j of a request at offset j % page_size of the physical
 * page that its page table lists for logical page j / page_size.  Here the
 * flat buffer [n_layers, size, ...] is that page view with
 * size = n_pages * page_size, so position j of the request on table row r
 * lives in slot
 *     req_to_token[r, j / page_size] * page_size + j % page_size,
 * and out_cache_loc keeps naming flat slots.  page_size 0 or 1: one-token
 * pages, req_to_token holds slots (the formula with page_size 1).
 * page_size > 1 must be a power of two (<= 65536) dividing size; then
 * req_to_token is [num_reqs, ceil(max_ctx_len / page_size)] of page ids. */
typedef struct {
  void *k_buffer;               /* device, [n_layers, size, n_kv_heads, head_dim] */
  void *v_buffer;               /* device, same shape and dtype                   */
  const int32_t *req_to_token;  /* device, [num_reqs, ceil(max_ctx_len / page_size)],
                                   row-major: slots (page_size 1) or page ids     */
  int64_t n_layers;
  int64_t size;                 /* slots per layer (a multiple of page_size)      */
  int64_t num_reqs;
  int64_t max_ctx_len;          /* logical positions a table row can address      */
  int32_t n_kv_heads;
  int32_t head_dim;
  pkv_dtype dtype;
  int32_t page_size;            /* tokens per page; 0 and 1 both mean one token   */
  int32_t v_head_dim;           /* width of the value rows; 0 means head_dim.  An
                                   MLA-shaped layer (v1.3.3 -> v1.3.4 compare page,
                                   class MLA) has keys of qk_nope_head_dim +
                                   qk_rope_head_dim = head_dim dims and values of
                                   v_head_dim: v_buffer is then
                                   [n_layers, size, n_kv_heads, v_head_dim]      */
  int32_t load_policy;          /* pkv_load_policy; 0 (zeroed struct): AUTO      */
} pkv_pool;

/* One step's KVCache metadata (same section).  Arrays are device pointers;
 * n_new, max_len and max_q_len are host values (max_len exists so that no
 * device->host read is needed to size the decode launch).  For decode,
 * max_len may be any bound of seq_lens up to max_ctx_len, not only their
 * maximum: the kernels read seq_lens from device memory, so a captured graph
 * can replay steps whose lengths (and out_cache_loc, position_ids) the
 * caller advances in place between replays.  A decode length that outgrows
 * the bound is still attended whole (the last split takes the keys past
 * num_splits times the split size, more slowly); a length past max_ctx_len
 * cannot be addressed through the table, and every decode entry point then
 * returns NaN for all heads of that request instead of reading anything. */
typedef struct {
  int32_t batch;
  const int32_t *req_pool_indices;  /* [batch] row of req_to_token per request        */
  const int32_t *seq_lens;          /* [batch] context length incl. this step's tokens */
  const int32_t *kv_indptr;         /* [batch+1] exclusive prefix sum of seq_lens      */
  const int32_t *qo_indptr;         /* [batch+1] exclusive prefix sum of q_lens; decode may pass NULL */
  const int32_t *out_cache_loc;     /* [n_new] write slots in qo order                 */
  int64_t n_new;                    /* total new tokens (decode: batch)                */
  int32_t max_len;                  /* max(seq_lens), or for decode any bound of them  */
  int32_t max_q_len;                /* max(q_lens) (decode: 1)                         */
  const int32_t *prefill_order;     /* [batch] or NULL: order in which prefill takes the
                                       requests (a permutation of 0..batch-1, e.g. the
                                       one pkv_build_step returns); affects speed only */
  const int32_t *prefill_blocks;    /* [2 * n_prefill_blocks] or NULL: the prefill launch
                                       schedule from pkv_prefill_blocks for this step and
                                       head counts; prefill then launches exactly these
                                       row blocks (prefill_order is not used) */
  int64_t n_prefill_blocks;         /* host: entries (pairs) of prefill_blocks              */
} pkv_step;

/* Human-readable name of a status. Never NULL. */
const char *pkv_status_string(pkv_status s);

/* hipError_t of the most recent PKV_ERR_HIP returned on the calling thread. */
int32_t pkv_last_hip_error(void);

/* ------------------------------------------------------------------------
 * Step metadata, host side ("Inference" guide, section "KVCache System":
 * kv_indptr and qo_indptr are prefix sums of seq_lens and of the per-request
 * new-token counts, computed once per step; out_cache_loc holds the write
 * slots of the forward; max_len = max(seq_lens)).
 *
 * All pointers are HOST memory.  Inputs: batch requests with table rows
 * req_pool_indices, context lengths seq_lens (this step's tokens included)
 * and new-token counts q_lens (NULL means 1 each, i.e. decode); the host
 * copy of req_to_token (rows of ceil(max_ctx_len / page_size) entries;
 * page_size as in pkv_pool, 0 meaning 1).  Request b's new tokens are its
 * last q_len_b logical positions, so its t-th new token is written to the
 * slot of position seq_len_b - q_len_b + t (pkv_pool's formula).
 * PKV_ERR_SHAPE when page_size is not 0, 1 or a power of two <= 65536.
 * Outputs: kv_indptr[batch+1], qo_indptr[batch+1], out_cache_loc (capacity
 * out_cache_loc_cap entries, filled in qo order), *n_new, *max_len,
 * *max_q_len, and, when prefill_order is not NULL, prefill_order[batch]: the
 * requests sorted by seq_len, longest first (ties in batch order), a
 * processing order for pkv_paged_prefill that starts the heaviest work
 * first.  Returns PKV_ERR_BAD_METADATA (outputs unspecified) when a
 * row, length or new-token count is out of range, PKV_ERR_SHAPE when
 * out_cache_loc_cap is too small.
 * ---------------------------------------------------------------------- */
pkv_status pkv_build_step(int32_t batch, const int32_t *req_pool_indices,
                          const int32_t *seq_lens, const int32_t *q_lens,
                          const int32_t *req_to_token, int64_t num_reqs,
                          int64_t max_ctx_len, int32_t page_size, int32_t *kv_indptr,
                          int32_t *qo_indptr, int32_t *out_cache_loc,
                          int64_t out_cache_loc_cap, int64_t *n_new,
                          int32_t *max_len, int32_t *max_q_len, int32_t *prefill_order);

/* Host: the logical position of every new token of a step, in qo order
 * (the rows of the rotary table its query and key use; "Inference" guide,
 * section "Rotary Embedding Backend": the table is indexed by
 * position_ids).  Request b's new tokens are its last q_len_b positions:
 * token t sits at seq_len_b - q_len_b + t.  All pointers are HOST memory;
 * q_lens NULL means one new token per request (decode).  Writes *n_new
 * entries of position_ids (capacity `capacity`).  PKV_ERR_BAD_METADATA when
 * a q_len is negative or above its seq_len, PKV_ERR_SHAPE when capacity is
 * too small. */
pkv_status pkv_build_positions(int32_t batch, const int32_t *seq_lens, const int32_t *q_lens,
                               int32_t *position_ids, int64_t capacity, int64_t *n_new);

/* Host: the prefill launch schedule of a step (affects speed only).  The
 * prefill kernel gives each workgroup one row block: up to
 * PKV_PREFILL_BLOCK_ROWS query rows of one request, rows enumerating (new
 * token t, query head g of a kv-head's group) as t * G + g, G = n_heads /
 * n_kv_heads.  This lists every non-empty row block as a pair (request, row
 * block index) in launch order: requests in the given order (order NULL:
 * batch order; pkv_build_step's prefill_order puts the longest contexts
 * first), and within a request the blocks of its last rows (the most keys
 * under the causal mask) first.  Passed to pkv_paged_prefill through
 * pkv_step.prefill_blocks, it launches no workgroup for rows that do not
 * exist (without it the grid covers max_q_len rows of every request).
 * All pointers are HOST memory; q_lens[b] new tokens of request b; blocks
 * has room for `capacity` pairs; *n_blocks receives the count.
 * PKV_ERR_SHAPE for bad head counts, a negative q_len or too small a
 * capacity; PKV_ERR_BAD_METADATA when order is not a permutation. */
#define PKV_PREFILL_BLOCK_ROWS 256
pkv_status pkv_prefill_blocks(int32_t batch, const int32_t *q_lens, const int32_t *order,
                              int32_t n_heads, int32_t n_kv_heads, int32_t *blocks,
                              int64_t capacity, int64_t *n_blocks);

/* Checked mode: validates HOST copies of one step's metadata against a pool
 * of `size` slots.  Accepts (PKV_OK) iff every request row is in
 * [0, num_reqs), every seq_len in [1, max_ctx_len], every q_len in
 * [0, seq_len], kv_indptr / qo_indptr are the exclusive prefix sums of the
 * lengths (qo_indptr NULL means decode: q_len 1 each), every slot read (of
 * positions 0 .. seq_len_b-1) lies in [0, size) (with pages: every page id
 * read lies in [0, size / page_size)), the write slots are pairwise
 * distinct, in [0, size), and equal the slot of their token's logical
 * position, and prefill_order (NULL: not checked) is a permutation of
 * 0..batch-1.  Else PKV_ERR_BAD_METADATA.  page_size as in pkv_pool
 * (PKV_ERR_SHAPE when invalid or not dividing size). */
pkv_status pkv_validate_step(int64_t size, int64_t num_reqs, int64_t max_ctx_len,
                             int32_t page_size, const int32_t *req_to_token, int32_t batch,
                             const int32_t *req_pool_indices, const int32_t *seq_lens,
                             const int32_t *kv_indptr, const int32_t *qo_indptr,
                             const int32_t *out_cache_loc, int64_t n_new,
                             const int32_t *prefill_order);

/* ------------------------------------------------------------------------
 * K/V write ("Inference" guide, section "KVCache System": the attention layer
 * stores this forward's keys with k_buffer[layer_id, out_cache_loc] = k, and
 * likewise v; section "Attention Backend": both backends write before they
 * attend).
 *
 * k_new, v_new: device, [n_new, n_kv_heads, head_dim], pool dtype.
 * out_cache_loc: device int32 [n_new], pairwise distinct slots in [0, size).
 * Row i of k_new / v_new is copied bit for bit to slot out_cache_loc[i] of
 * layer layer_id; no other byte of the pool changes.  n_new == 0 is a no-op.
 * ---------------------------------------------------------------------- */
pkv_status pkv_kv_store(const pkv_pool *pool, int32_t layer_id, const void *k_new,
                        const void *v_new, const int32_t *out_cache_loc, int64_t n_new,
                        void *stream /* hipStream_t */);

/* ------------------------------------------------------------------------
 * Decode workspace (commit history of tests/inference/test_cache.py: the
 * per-split partial outputs and (max, sum) pairs live in buffers the caller
 * allocates once and passes to every step).
 *
 * Bytes needed by pkv_paged_decode / pkv_paged_decode_merge for up to
 * max_batch requests, n_heads query heads and num_splits splits.  Layout
 * (internal, documented for debugging): o_part fp32 [batch, n_heads,
 * num_splits, head_dim], then ml_part fp32 [batch, n_heads, num_splits, 2]
 * holding (m, l): m = running max of the base-2 scaled score
 * (score * sm_scale * log2 e), l = sum of 2^(scaled score - m); o_part is
 * normalised by l.  Empty splits hold (-inf, 0) and o = 0.
 * Returns 0 for non-positive arguments.
 * ---------------------------------------------------------------------- */
size_t pkv_decode_workspace_bytes(int32_t max_batch, int32_t n_heads, int32_t head_dim,
                                  int32_t num_splits);

/* Host-only split-count heuristic (no device access, no sync).  From the
 * batch, head counts, the host max_len and the step's total context tokens
 * (kv_indptr[batch]; <= 0 means batch * max_len) it picks num_splits for
 * pkv_paged_decode: for equal lengths about one long-running wavefront per
 * SIMD, for ragged lengths about four splits per SIMD of at most 512 tokens
 * (an odd count) so the device balances the load; clamped to
 * [1, max_splits]. */
int32_t pkv_decode_pick_splits(int32_t batch, int32_t n_kv_heads, int32_t n_heads,
                               int32_t max_len, int64_t total_len, int32_t max_splits);

/* Host, no device access: whether the bf16 matrix-core decode kernels
 * (pkv_paged_decode, pkv_paged_decode_store, pkv_paged_decode_rope_store)
 * read K/V rows with non-temporal loads for a decode step of `batch`
 * requests with max_len as pkv_step.max_len on this pool, under its
 * load_policy (see pkv_load_policy): 1 non-temporal, 0 cached, -1 for a null
 * pool or invalid fields.  Affects speed only. */
int32_t pkv_decode_load_kind(const pkv_pool *pool, int32_t batch, int32_t max_len);

/* ------------------------------------------------------------------------
 * Split-KV paged decode ("Inference" guide, section "KV Cache": the single
 * new query row of each request attends over all its cached keys,
 * o = sum_j softmax(q . k_j * sm_scale) v_j; section "Attention Backend":
 * req_to_token is the page table (one-token pages there; any page_size of
 * pkv_pool here) and the kernel gathers
 * K/V itself; commit history of tests/inference/test_cache.py: per-split
 * partial outputs in a caller-owned workspace).
 *
 * q: device [batch, n_heads, head_dim], pool dtype.  Query head h reads
 * kv-head h / (n_heads / n_kv_heads).  Request b attends to logical keys
 * 0 .. seq_lens[b]-1 (the token written this step included; write it with
 * pkv_kv_store first) of layer layer_id.  Keys are split into num_splits
 * contiguous logical ranges of ceil(max_len / num_splits) tokens (rounded up
 * to a multiple of 16; the last range also takes any keys beyond
 * num_splits such ranges); each split's (m, l, o) partial goes to the workspace
 * (layout above).  Call pkv_paged_decode_merge to form the output.
 * Errors: PKV_ERR_WORKSPACE_TOO_SMALL when ws_bytes <
 * pkv_decode_workspace_bytes(batch, n_heads, head_dim, num_splits).
 * ---------------------------------------------------------------------- */
pkv_status pkv_paged_decode(const pkv_pool *pool, int32_t layer_id, const pkv_step *step,
                            const void *q, int32_t n_heads, float sm_scale,
                            int32_t num_splits, void *workspace, size_t ws_bytes,
                            void *stream /* hipStream_t */);

/* Merge of the split partials written by pkv_paged_decode with the same
 * batch, n_heads, head_dim and num_splits (same commit history entry): with
 * M = max_s m_s and w_s = l_s 2^(m_s - M), out = sum_s w_s o_s / sum_s w_s;
 * empty splits weigh 0.  out: device [batch, n_heads, head_dim] in out_dtype
 * (bf16 rounded to nearest even). */
pkv_status pkv_paged_decode_merge(int32_t batch, int32_t n_heads, int32_t head_dim,
                                  pkv_dtype out_dtype, int32_t num_splits,
                                  const void *workspace, size_t ws_bytes, void *out,
                                  void *stream /* hipStream_t */);

/* ------------------------------------------------------------------------
 * In-place advance of a decode step's device metadata to the next token
 * (commit history of the pages: decode metadata such as position_ids,
 * seq_lens and kv_indptr is updated in place from step to step instead of
 * being rebuilt, so that a captured graph can be replayed).  One launch:
 *   seq_lens[b] += 1; position_ids[b] = seq_lens[b] - 1 (if not NULL);
 *   out_cache_loc[b] = slot of position seq_lens[b] - 1 of table row
 *                      req_pool_indices[b] (pkv_pool's formula);
 *   kv_indptr[b] += b for b in [0, batch] (if not NULL).
 * All arrays are device int32 owned by the caller; the caller keeps every
 * length within max_ctx_len.  Past it, out_cache_loc[b] is clamped to the
 * slot of position max_ctx_len - 1 (a pkv_kv_store or pkv_rope_kv_store of
 * that step overwrites that token; the one- and two-launch decode steps skip
 * the write) and the decode entry points return NaN for the request (see
 * pkv_step).  The host max_len of the step should bound the lengths the next
 * steps reach (longer ones are attended correctly, but the last split takes
 * the excess alone).  batch == 0 is a no-op.
 * Errors: PKV_ERR_NULL (missing seq_lens / req_pool_indices / out_cache_loc),
 * PKV_ERR_SHAPE (batch < 0).
 * ---------------------------------------------------------------------- */
pkv_status pkv_decode_advance(const pkv_pool *pool, int32_t batch, const int32_t *req_pool_indices,
                              int32_t *seq_lens, int32_t *kv_indptr, int32_t *out_cache_loc,
                              int32_t *position_ids, void *stream);

/* ------------------------------------------------------------------------
 * Rotary embedding of one forward's new tokens fused with their K/V write
 * ("Inference" guide, section "Rotary Embedding Backend": freqs_cis
 * [max_len, dim/2, 2] f32 holds [cos, sin] pairs, the rows used are those of
 * position_ids, and adjacent elements (2j, 2j+1) form one complex number
 * multiplied by cos + i sin; section "KV Cache": keys are rotated before the
 * cache write, values are not rotated).  For every new token i at position
 * p = position_ids[i] and every pair j of every head row:
 *   (x[2j], x[2j+1]) -> (x[2j] c - x[2j+1] s, x[2j] s + x[2j+1] c),
 *   (c, s) = freqs_cis[p, j],
 * computed in fp32 and rounded once to the pool dtype (bf16: to nearest,
 * ties to even).  Queries: q -> q_out (q_out may equal q).  Keys: the rotated
 * row i goes to slot out_cache_loc[i] of layer layer_id; values: v_new row i
 * is copied there bit for bit.  No other byte of the pool changes.
 * q, q_out: device [n_new, n_heads, head_dim]; k_new, v_new: device
 * [n_new, n_kv_heads, head_dim]; all in the pool dtype, 16-byte aligned.
 * position_ids, out_cache_loc: device int32 [n_new] (pkv_build_positions and
 * pkv_build_step give them in the same qo order).  freqs_cis: device f32
 * [max_pos, head_dim/2, 2], 16-byte aligned.  The caller guarantees positions
 * in [0, max_pos) (others read the nearest row) and distinct slots in
 * [0, size).  n_new == 0 is a no-op.
 * Errors: PKV_ERR_NULL (missing pointer), PKV_ERR_SHAPE (n_heads not a
 * positive multiple of n_kv_heads, max_pos <= 0, n_new < 0, misaligned
 * pointer), PKV_ERR_UNSUPPORTED (head_dim other than 64 / 128).
 * ---------------------------------------------------------------------- */
pkv_status pkv_rope_kv_store(const pkv_pool *pool, int32_t layer_id, const void *q, void *q_out,
                             int32_t n_heads, const void *k_new, const void *v_new,
                             const int32_t *position_ids, const float *freqs_cis,
                             int64_t max_pos, const int32_t *out_cache_loc, int64_t n_new,
                             void *stream);

/* The same write for MLA-shaped layers (v1.3.3 -> v1.3.4 compare page, class
 * MLA: queries and keys of qk_nope_head_dim + qk_rope_head_dim dims, the
 * rotation on the qk_rope part): only the last rope_dim dims of every query
 * and key row are rotated, pair j of that part by freqs_cis[p, j]
 * (freqs_cis: device f32 [max_pos, rope_dim / 2, 2]); the first
 * head_dim - rope_dim dims are copied unchanged; value rows (v_head_dim
 * wide) are copied.  k_new is [n_new, n_kv_heads, head_dim], v_new
 * [n_new, n_kv_heads, v_head_dim].  pkv_rope_kv_store is this call with
 * rope_dim = head_dim.  Errors: as pkv_rope_kv_store, plus PKV_ERR_SHAPE
 * when rope_dim is not in (0, head_dim] or not a multiple of 16 bytes of
 * elements (8 for bf16, 4 for f32). */
pkv_status pkv_rope_kv_store_partial(const pkv_pool *pool, int32_t layer_id, const void *q,
                                     void *q_out, int32_t n_heads, const void *k_new,
                                     const void *v_new, const int32_t *position_ids,
                                     const float *freqs_cis, int64_t max_pos, int32_t rope_dim,
                                     const int32_t *out_cache_loc, int64_t n_new, void *stream);

/* ------------------------------------------------------------------------
 * One decode step in one launch ("Inference" guide, section "KVCache System":
 * the new token's K/V are written at out_cache_loc; section "Attention
 * Backend": decode then attends the paged cache; commit history of
 * tests/inference/test_cache.py: split partials in a caller-owned workspace
 * merged by log-sum-exp).  Computes exactly what pkv_kv_store (of the step's
 * batch new tokens) followed by pkv_paged_decode and pkv_paged_decode_merge
 * computes, for decode steps (one new token per request: step->n_new ==
 * batch, qo_indptr unused):
 *   k_buffer[layer, out_cache_loc[b]] = k_new[b] (same for v), then
 *   out[b, h] = sum_j softmax_j(q[b,h] . k_j * sm_scale) v_j over the
 *   seq_lens[b] keys of request b, the new one included.
 * k_new / v_new: device [batch, n_kv_heads, head_dim], pool dtype.  q, out:
 * device [batch, n_heads, head_dim], pool dtype.
 * For bf16 pools with head_dim 128 this is one kernel: each split is taken by
 * a four-wave workgroup, the new token's rows are read from k_new / v_new
 * (and written to the pool by one workgroup), and the last workgroup of each
 * (request, kv-head) to finish merges that kv-head's heads.  Requirements of
 * that path: out_cache_loc[b] is the slot of position seq_lens[b] - 1 of
 * request b and no other position read in this step maps to it (fresh slots,
 * as pkv_validate_step checks for duplicates); sync points to sync_len >=
 * batch * n_heads int32 counters that are zero before the first call (each
 * call leaves them zero; re-zero them after a failed call).  Other shapes run
 * the three launches (sync unused).
 * workspace: pkv_decode_workspace_bytes(batch, n_heads, head_dim, num_splits)
 * bytes, layout as for pkv_paged_decode.  num_splits: see
 * pkv_decode_step_pick_splits.
 * Errors: as pkv_paged_decode, plus PKV_ERR_NULL for missing k_new / v_new /
 * out / sync / out_cache_loc and PKV_ERR_SHAPE for n_new != batch or a short
 * sync buffer.
 * ---------------------------------------------------------------------- */
pkv_status pkv_paged_decode_step(const pkv_pool *pool, int32_t layer_id, const pkv_step *step,
                                 const void *q, const void *k_new, const void *v_new,
                                 int32_t n_heads, float sm_scale, int32_t num_splits,
                                 void *workspace, size_t ws_bytes, int32_t *sync,
                                 int64_t sync_len, void *out, void *stream /* hipStream_t */);

/* ----------------------------------------------------------------------
 * One decode step in two launches (same sources and the same result as
 * pkv_paged_decode_step): the split attention of pkv_paged_decode with the
 * new-token K/V write folded in, then pkv_paged_decode_merge into out.
 *   k_buffer[layer, out_cache_loc[b]] = k_new[b] (same for v), then
 *   out[b, h] = sum_j softmax_j(q[b,h] . k_j * sm_scale) v_j over the
 *   seq_lens[b] keys of request b, the new one included.
 * Decode steps only: step->n_new == batch (one new token per request,
 * qo_indptr unused).  k_new / v_new: device [batch, n_kv_heads, head_dim],
 * pool dtype; q, out: device [batch, n_heads, head_dim], pool dtype.
 * For bf16 pools with head_dim 128 the split kernel attends the new token's
 * rows straight from k_new / v_new and one wavefront per kv-head writes them
 * to the pool; this needs out_cache_loc[b] to be the slot of position
 * seq_lens[b] - 1 of request b with no other position read in this step
 * mapped to it (fresh slots, as pkv_validate_step checks for duplicates).
 * Other shapes run pkv_kv_store, pkv_paged_decode and the merge.
 * workspace / num_splits: as for pkv_paged_decode (pkv_decode_pick_splits,
 * pkv_decode_workspace_bytes); no counters are needed.
 * Errors: as pkv_paged_decode, plus PKV_ERR_NULL for missing k_new / v_new /
 * out / out_cache_loc and PKV_ERR_SHAPE for n_new != batch.
 * ---------------------------------------------------------------------- */
pkv_status pkv_paged_decode_store(const pkv_pool *pool, int32_t layer_id, const pkv_step *step,
                                  const void *q, const void *k_new, const void *v_new,
                                  int32_t n_heads, float sm_scale, int32_t num_splits,
                                  void *workspace, size_t ws_bytes, void *out, void *stream);

/* ----------------------------------------------------------------------
 * The decode step of pkv_rope_kv_store followed by pkv_paged_decode_store,
 * in two launches ("Inference" guide, section "Rotary Embedding Backend":
 * the query and the new key are rotated by the freqs_cis row of their
 * position before the cache write and the attention; section "KV Cache";
 * section "Attention Backend").  q and k_new arrive unrotated:
 *   q'[b] = rot(q[b], position_ids[b]), k'[b] = rot(k_new[b], position_ids[b])
 *   k_buffer[layer, out_cache_loc[b]] = k'[b], v_buffer[...] = v_new[b],
 *   out[b, h] = sum_j softmax_j(q'[b,h] . k_j * sm_scale) v_j
 * over the seq_lens[b] keys of request b, the new one included, with rot
 * the rotation of pkv_rope_kv_store (fp32, rounded once to bf16), so the
 * output and the pool equal those of the two calls bit for bit; q' is not
 * written anywhere.  Decode steps only (step->n_new == batch).  Pools of
 * bf16 with head_dim and v_head_dim 128 and at most 16 query heads per
 * kv-head; out_cache_loc[b] must be the slot of position seq_lens[b] - 1 of
 * request b, with no other position read in this step mapped to it (the new
 * rows are written to the pool before they are attended).
 * position_ids: device int32 [batch]; freqs_cis: device f32
 * [max_pos, 64, 2], 16-byte aligned; workspace / num_splits as for
 * pkv_paged_decode_store.
 * Errors: as pkv_paged_decode_store and pkv_rope_kv_store, plus
 * PKV_ERR_UNSUPPORTED for other pool shapes or more than 16 query heads per
 * kv-head.
 * ---------------------------------------------------------------------- */
pkv_status pkv_paged_decode_rope_store(const pkv_pool *pool, int32_t layer_id,
                                       const pkv_step *step, const void *q, const void *k_new,
                                       const void *v_new, const int32_t *position_ids,
                                       const float *freqs_cis, int64_t max_pos, int32_t n_heads,
                                       float sm_scale, int32_t num_splits, void *workspace,
                                       size_t ws_bytes, void *out, void *stream);

/* ----------------------------------------------------------------------
 * The decode step of pkv_paged_decode_store without a caller workspace, for
 * callers that cannot allocate device memory (code under graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, result
 * and kernels as pkv_paged_decode_store, minus workspace / ws_bytes: the
 * split partials go to a static device array of PKV_NOALLOC_SCRATCH_BYTES
 * bytes that the library holds on every device it runs on until the process
 * ends (its address is looked up on the first call on each device).  Nothing
 * is allocated or freed.  Every call on a device shares that device's array:
 * calls that overlap on one device (other streams, other threads) race and
 * must be serialised by the caller; calls in order on one stream do not
 * (each call rewrites every partial it reads).
 * Errors: as pkv_paged_decode_store, plus PKV_ERR_SCRATCH_LIMIT when
 * pkv_decode_workspace_bytes(batch, n_heads, head_dim, num_splits) exceeds
 * PKV_NOALLOC_SCRATCH_BYTES (nothing is launched), and PKV_ERR_HIP when the
 * array's address cannot be obtained.
 * ---------------------------------------------------------------------- */
#define PKV_NOALLOC_SCRATCH_BYTES (32u << 20)
pkv_status pkv_paged_decode_store_noalloc(const pkv_pool *pool, int32_t layer_id,
                                          const pkv_step *step, const void *q, const void *k_new,
                                          const void *v_new, int32_t n_heads, float sm_scale,
                                          int32_t num_splits, void *out, void *stream);

/* ------------------------------------------------------------------------
 * Decode with shared prefixes ("Inference" guide, section "KVCache System":
 * the allocator and prefix cache let requests share the slots of a common
 * prompt prefix; commit history of tests/inference/test_cache.py: request
 * mappings are rebuilt for cached prefix pages).  When several requests of a
 * step read the same slots for their first P positions, the decode step can
 * read those keys once per group instead of once per request: one launch
 * attends every group's shared keys with all members' query heads together,
 * the split kernel attends each request's keys from kv_start[b] = P on, and
 * the merge combines both.  The result is the same function as
 * pkv_paged_decode_store (the same per-head softmax over all seq_lens[b]
 * keys); only the order of the fp32 sums differs.
 *
 * A group record is PKV_PREFIX_GROUP_INTS int32: [P, m, b_0 .. b_{m-1}, 0 ..]
 * with 2 <= m <= PKV_PREFIX_GROUP_MAX members (batch indices) whose table
 * rows agree on every entry of positions 0 .. P-1 and whose seq_lens exceed
 * P (each request's newest position stays its own).
 * ---------------------------------------------------------------------- */
#define PKV_PREFIX_GROUP_MAX 16
#define PKV_PREFIX_GROUP_INTS (2 + PKV_PREFIX_GROUP_MAX)

typedef struct {
  const int32_t *groups;    /* device [n_groups * PKV_PREFIX_GROUP_INTS] group records      */
  const int32_t *kv_start;  /* device [batch]: P of the request's group, 0 for none          */
  int32_t n_groups;
  int32_t max_prefix;       /* host: largest P                                              */
  int32_t max_members;      /* host: largest member count                                   */
  int32_t max_suffix;       /* host: bound of seq_lens[b] - kv_start[b] over the batch      */
} pkv_prefix_groups;

/* Host: the prefix groups of a decode step, from HOST copies of its metadata
 * and table (page_size as in pkv_pool).  Requests whose first table entries
 * agree are grouped: each group takes a lead (the longest such request,
 * the earliest on ties) and the requests sharing the most leading positions with it
 * (at most PKV_PREFIX_GROUP_MAX members), with P the smallest shared range
 * among them, chosen to maximise (members - 1) * P; groups with P <
 * min_prefix are not formed, and the other requests are grouped again among
 * themselves.  A request's shared range never includes its last position.
 * Writes *n_groups records to groups (capacity groups_cap records),
 * kv_start[batch] (P or 0), and the host bounds *max_prefix, *max_members,
 * *max_suffix (max of seq_lens[b] - kv_start[b]).  Affects speed only: any
 * valid grouping, or none, gives the same result.
 * Errors: PKV_ERR_NULL, PKV_ERR_SHAPE (bad page size, too small a capacity),
 * PKV_ERR_BAD_METADATA (request row or length out of range). */
pkv_status pkv_decode_prefix_groups(int32_t batch, const int32_t *req_pool_indices,
                                    const int32_t *seq_lens, const int32_t *req_to_token,
                                    int64_t num_reqs, int64_t max_ctx_len, int32_t page_size,
                                    int32_t min_prefix, int32_t *groups, int64_t groups_cap,
                                    int64_t *n_groups, int32_t *kv_start, int32_t *max_prefix,
                                    int32_t *max_members, int32_t *max_suffix);

/* The decode step of pkv_paged_decode_store (new-token K/V write, attention,
 * merge; same arguments and contract) with the shared prefixes of `groups`
 * (device arrays from pkv_decode_prefix_groups for this step's metadata and
 * tables) read once per group.  num_splits splits cover each request's own
 * keys [kv_start[b], seq_lens[b]) (split size from groups->max_suffix; the
 * last split takes any excess), prefix_splits splits each group's shared
 * keys.  workspace: pkv_decode_workspace_bytes(batch, n_heads, head_dim,
 * num_splits + prefix_splits) bytes.  Three launches (shared keys, own keys
 * with the K/V write, merge) for bf16 pools with head_dim 128; with groups
 * NULL or n_groups 0, or other pools, this is pkv_paged_decode_store.
 * Errors: as pkv_paged_decode_store, plus PKV_ERR_SHAPE for prefix_splits
 * outside [1, 65535] or inconsistent host bounds in groups. */
pkv_status pkv_paged_decode_shared(const pkv_pool *pool, int32_t layer_id, const pkv_step *step,
                                   const pkv_prefix_groups *groups, const void *q,
                                   const void *k_new, const void *v_new, int32_t n_heads,
                                   float sm_scale, int32_t num_splits, int32_t prefix_splits,
                                   void *workspace, size_t ws_bytes, void *out, void *stream);

/* Host-only split count for pkv_paged_decode_step: the single-wave choice of
 * pkv_decode_pick_splits divided by four (each split of the fused step is
 * taken by four wavefronts), clamped to [1, max_splits]. */
int32_t pkv_decode_step_pick_splits(int32_t batch, int32_t n_kv_heads, int32_t n_heads,
                                    int32_t max_len, int64_t total_len, int32_t max_splits);

/* ------------------------------------------------------------------------
 * Ragged paged prefill ("Inference" guide, section "Attention Backend": after
 * the K/V write, a ragged-batch kernel reads K/V straight from the flat pool
 * through req_to_token, with each request's query and key counts taken from
 * qo_indptr and kv_indptr).
 *
 * q, out: device [n_new, n_heads, head_dim] bf16, packed in qo order.
 * Request i owns query rows qo_indptr[i] .. qo_indptr[i+1]-1 and
 * kv_len_i = kv_indptr[i+1] - kv_indptr[i] keys; its t-th new token sits at
 * logical position p_i + t with p_i = kv_len_i - q_len_i.  With causal != 0
 * that token attends keys 0 .. p_i + t (mask aligned to the end of the
 * context); with causal == 0 it attends all kv_len_i keys.  QK^T and PV run
 * as bf16 matrix-core tiles with fp32 accumulation; the softmax weights are
 * rounded to bf16 before the PV product.  Uses step->max_q_len (host) to
 * size the launch, or, when step->prefill_blocks is set, launches exactly
 * step->n_prefill_blocks row blocks per kv-head (the list must be
 * pkv_prefill_blocks' for this step's q_lens and these head counts; like
 * other device metadata it is not read on the host).  Only PKV_BF16 pools
 * are accepted (else PKV_ERR_DTYPE);
 * sm_scale must be finite and > 0 (else PKV_ERR_SHAPE).
 * ---------------------------------------------------------------------- */
pkv_status pkv_paged_prefill(const pkv_pool *pool, int32_t layer_id, const pkv_step *step,
                             const void *q, int32_t n_heads, float sm_scale,
                             int32_t causal, void *out, void *stream /* hipStream_t */);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */

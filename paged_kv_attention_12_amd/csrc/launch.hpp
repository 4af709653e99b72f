// Internal launch interface between the C ABI (pkv_api.cpp) and the kernels.
// Arguments here are already validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Records e as the calling thread's last HIP error (pkv_last_hip_error) and
// returns PKV_ERR_HIP (as an int: pkv_status lives in the C header).
int note_hip_error(hipError_t e);

struct KvStoreArgs {
  void *k_layer;              // k_buffer + layer_id * size * row_elems (bytes as char*)
  void *v_layer;
  const void *k_new;          // [n_new, row_bytes]
  const void *v_new;
  const int32_t *out_cache_loc;
  int64_t n_new;
  int64_t size;
  int32_t row_bytes;          // key row: n_kv_heads * head_dim * sizeof(dtype)
  int32_t v_row_bytes;        // value row: n_kv_heads * v_head_dim * sizeof(dtype) (<= row_bytes)
};
hipError_t launch_kv_store(const KvStoreArgs &a, hipStream_t stream);

// In-place advance of a decode step's metadata to the next token.
struct AdvanceArgs {
  const int32_t *req_to_token;      // slot table, or page table when page_shift > 0
  int64_t max_ctx_len;              // logical positions a table row addresses
  int64_t table_stride;             // entries per table row: ceil(max_ctx_len / page)
  int32_t page_shift;               // log2(tokens per page)
  const int32_t *req_pool_indices;  // [batch]
  int32_t *seq_lens;                // [batch]
  int32_t *kv_indptr;               // [batch + 1] or null
  int32_t *out_cache_loc;           // [batch]
  int32_t *position_ids;            // [batch] or null
  int32_t batch;
};
hipError_t launch_decode_advance(const AdvanceArgs &a, hipStream_t stream);

struct DecodeArgs {
  const void *k_layer;        // first element of layer layer_id
  const void *v_layer;
  const int32_t *req_to_token;      // slot table, or page table when page_shift > 0
  int64_t max_ctx_len;              // logical positions a table row addresses
  int64_t table_stride;             // entries per table row: ceil(max_ctx_len / page)
  int32_t page_shift;               // log2(tokens per page)
  const int32_t *req_pool_indices;
  const int32_t *seq_lens;
  const void *q;              // [batch, n_heads, head_dim]
  float *o_part;              // [batch, n_heads, num_splits, head_dim]
  float *ml_part;             // [batch, n_heads, num_splits, 2]
  int32_t batch;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t group;              // n_heads / n_kv_heads
  int32_t n_chunks;           // head chunks per kv-head (set by the launcher)
  int32_t heads_per_chunk;    // query heads per chunk (set by the launcher)
  int32_t num_splits;
  int32_t chunk;              // tokens per split (multiple of 16)
  float scale_log2;           // sm_scale * log2(e)
  // Shared-prefix decode (matrix-core split kernel only): request b's splits
  // cover keys [kv_start[b], seq_lens[b]) (null: from 0), and partial rows
  // hold split_stride splits (num_splits when no prefix partials follow).
  const int32_t *kv_start;
  int32_t split_stride;
  // Splits with no keys leave their partial unwritten (the merge is told
  // which splits hold keys); 0: every split writes one.
  int32_t skip_empty;
  // Matrix-core split kernels: K/V rows read with non-temporal loads.
  int32_t stream_rows;
};
// dtype: 0 = f32, 1 = bf16.  head_dim: key width; v_head_dim: value width.
hipError_t launch_paged_decode(const DecodeArgs &a, int dtype, int head_dim, int v_head_dim,
                               hipStream_t stream);
// Shapes the matrix-core split kernel takes: bf16, values 128 wide, keys 128
// or 192 wide (the split-with-write and shared-prefix paths need them).
bool decode_mfma_shape(int dtype, int head_dim, int v_head_dim);

// One fused decode step (bf16, head_dim 128): new-token K/V write, split
// attention and merge in one launch.
struct StepArgs {
  DecodeArgs d;               // o_part / ml_part: the decode workspace
  const void *k_new;          // [batch, n_kv_heads, head_dim]
  const void *v_new;
  void *k_layer_w;            // d.k_layer, writable
  void *v_layer_w;
  const int32_t *out_cache_loc;  // [batch]
  int32_t *sync;              // [batch * tasks] ticket counters, zero between calls
  void *out;                  // [batch, n_heads, head_dim] bf16
  int32_t tasks;              // kv-heads x head chunks (set by the launcher)
  // Rotary embedding folded in (launch_decode_split_rope only): q and k_new
  // arrive unrotated and are turned by row position_ids[b] of freqs.
  const int32_t *position_ids;  // [batch]
  const float *freqs;           // [max_pos, head_dim / 2, 2]: [cos, sin]
  int64_t max_pos;
};
hipError_t launch_decode_step(const StepArgs &a, hipStream_t stream);
// The split attention of one decode step with the new-token K/V write folded
// in (bf16, head_dim 128); sync, out and tasks are not used.  The merge is a
// separate launch.
hipError_t launch_decode_split_store(const StepArgs &a, int head_dim, hipStream_t stream);
// The same with the rotary embedding of q and k_new folded in (bf16, keys
// and values 128 wide): every wavefront turns its query rows, and the new
// key row is turned before it is attended and written.
hipError_t launch_decode_split_rope(const StepArgs &a, hipStream_t stream);

// Rotary embedding of the new tokens fused with their K/V write.
struct RopeArgs {
  const void *q;              // [n_new, n_heads, head_dim], pool dtype
  void *q_out;                // same shape; may equal q
  const void *k_new;          // [n_new, n_kv_heads, head_dim]
  const void *v_new;
  void *k_layer;              // layer layer_id of the pool (writable)
  void *v_layer;
  const int32_t *position_ids;  // [n_new]
  const float *freqs;         // [max_pos, head_dim / 2, 2]: [cos, sin]
  int64_t max_pos;
  const int32_t *out_cache_loc;  // [n_new]
  int64_t n_new;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;           // query / key rows
  int32_t v_head_dim;         // value rows
  int32_t rope_dim;           // rotated part: the last rope_dim dims of each row
};
// dtype: 0 = f32, 1 = bf16
hipError_t launch_rope_kv_store(const RopeArgs &a, int dtype, hipStream_t stream);

struct MergeArgs {
  const float *o_part;
  const float *ml_part;
  void *out;                  // [batch, n_heads, head_dim]
  int32_t rows;               // batch * n_heads
  int32_t num_splits;         // splits of every row
  // Shared-prefix decode: rows hold `stride` splits; a request with
  // kv_start[b] > 0 also has prefix_splits prefix partials after its
  // num_splits own ones (null kv_start: stride == num_splits, none).
  const int32_t *kv_start;
  int32_t stride;
  int32_t n_heads;
  int32_t prefix_splits;
  // When not null, only the splits holding keys are read: own splits from
  // kv_start (or 0) in steps of chunk up to seq_lens, prefix splits in steps
  // of prefix_chunk below kv_start (lengths past max_ctx_len: all splits).
  const int32_t *seq_lens;
  int32_t chunk;
  int32_t prefix_chunk;
  int64_t max_ctx_len;
};

// Shared-prefix decode: a group's members share the slots of their first P
// positions; the group record (PKV_PREFIX_GROUP_INTS int32 on the device) is
// [P, m, b_0 .. b_{m-1}].  One launch attends every group's shared keys with
// the members' query heads as matrix-core columns and writes each member's
// prefix partials after its own splits.
struct PrefixArgs {
  DecodeArgs d;               // chunk: prefix split size; num_splits: the
                              // members' own splits (prefix partials follow)
  const int32_t *groups;
  int32_t n_groups;
  int32_t prefix_splits;
  int32_t group_ints;         // int32 per group record
  int32_t max_members;
};
hipError_t launch_decode_prefix(const PrefixArgs &a, hipStream_t stream);

// The shared-prefix attention of one decode step in one launch: prefix
// workgroups first, then every request's own splits with the K/V write.
struct SharedArgs {
  StepArgs sfx;               // own keys from kv_start (d.kv_start set)
  PrefixArgs pfx;
  int32_t pfx_wx;             // workgroups per (group, prefix split)  (set by the launcher)
  int32_t sfx_wx;             // workgroups per (request, split)       (set by the launcher)
  int32_t pfx_blocks;         // prefix workgroups                      (set by the launcher)
};
hipError_t launch_decode_shared(const SharedArgs &a, hipStream_t stream);
hipError_t launch_decode_merge(const MergeArgs &a, int dtype, int head_dim, hipStream_t stream);

struct PrefillArgs {
  const void *k_layer;
  const void *v_layer;
  const int32_t *req_to_token;      // slot table, or page table when page_shift > 0
  int64_t max_ctx_len;              // logical positions a table row addresses
  int64_t table_stride;             // entries per table row: ceil(max_ctx_len / page)
  int32_t page_shift;               // log2(tokens per page)
  const int32_t *req_pool_indices;
  const int32_t *qo_indptr;
  const int32_t *kv_indptr;
  const int32_t *order;       // [batch] request processing order, or null
  const int32_t *blocks;      // [2 * n_blocks] (request, row block) launch list, or null
  int64_t n_blocks;
  const void *q;              // [n_new, n_heads, head_dim] bf16
  void *out;                  // [n_new, n_heads, head_dim] bf16
  int64_t pool_size;          // slots per layer
  int32_t batch;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t group;
  int32_t max_q_len;
  int32_t row_blocks;         // row blocks per request in the launch (set by the launcher)
  int32_t causal;
  float scale_log2;
};
// head_dim: query / key width; v_head_dim: value / output width.
hipError_t launch_paged_prefill(const PrefillArgs &a, int head_dim, int v_head_dim,
                                hipStream_t stream);
constexpr int kPrefillBlockRows = 256;  // query rows of one prefill workgroup

}  // namespace pkv

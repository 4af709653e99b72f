// C ABI of libpkv: argument checks, workspace sizing, split choice and kernel
// launches on the caller's stream.  Declarations and contracts: include/pkv.h.
#include "../../include/pkv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <unordered_set>
#include <vector>

#include "launch.hpp"

namespace {

thread_local int32_t g_last_hip_error = 0;

pkv_status hip_status(hipError_t e) {
  if (e == hipSuccess) return PKV_OK;
  g_last_hip_error = (int32_t)e;
  return PKV_ERR_HIP;
}

size_t dtype_bytes(pkv_dtype d) { return d == PKV_BF16 ? 2 : 4; }

bool dtype_ok(pkv_dtype d) { return d == PKV_F32 || d == PKV_BF16; }

// Token-range granularity of one split (rows per decode iteration divide it).
constexpr int32_t kSplitAlign = 16;

// log2 of a page size (0 and 1 both mean one-token pages); -1 when the size is
// not a power of two in [1, 65536].
int page_shift_of(int32_t page_size) {
  if (page_size == 0) return 0;
  for (int sh = 0; sh <= 16; ++sh)
    if (page_size == (1 << sh)) return sh;
  return -1;
}

// Entries per table row: one per page of up to max_ctx_len positions.
int64_t table_stride_of(int64_t max_ctx_len, int page_shift) {
  return (max_ctx_len + (int64_t(1) << page_shift) - 1) >> page_shift;
}

// Width of the value rows (0 in the pool: as wide as the keys).
int32_t v_dim(const pkv_pool *p) { return p->v_head_dim > 0 ? p->v_head_dim : p->head_dim; }

// Key / value widths the attention kernels take: equal widths of 64 or 128,
// or MLA-shaped keys of 192 with values of 128.
bool dims_ok(const pkv_pool *p) {
  const int32_t dk = p->head_dim, dv = v_dim(p);
  return (dk == dv && (dk == 64 || dk == 128)) || (dk == 192 && dv == 128);
}

pkv_status check_pool(const pkv_pool *p, int32_t layer_id) {
  if (!p || !p->k_buffer || !p->v_buffer || !p->req_to_token) return PKV_ERR_NULL;
  if (!dtype_ok(p->dtype)) return PKV_ERR_DTYPE;
  if (p->n_layers <= 0 || p->size <= 0 || p->num_reqs <= 0 || p->max_ctx_len <= 0 ||
      p->n_kv_heads <= 0 || p->head_dim <= 0 || p->v_head_dim < 0 || v_dim(p) > p->head_dim)
    return PKV_ERR_SHAPE;
  if (p->size > INT32_MAX) return PKV_ERR_SHAPE;  // slots are int32
  if (p->max_ctx_len > INT32_MAX) return PKV_ERR_SHAPE;  // positions are int32
  const int sh = page_shift_of(p->page_size);
  if (sh < 0 || p->size % (int64_t(1) << sh) != 0) return PKV_ERR_SHAPE;
  if (layer_id < 0 || layer_id >= p->n_layers) return PKV_ERR_SHAPE;
  if (p->load_policy < PKV_LOAD_AUTO || p->load_policy > PKV_LOAD_STREAM) return PKV_ERR_SHAPE;
  return PKV_OK;
}

// MI355X's last-level (Infinity) cache.
constexpr int64_t kLastLevelCacheBytes = int64_t(256) << 20;

// Whether the matrix-core decode kernels read K/V rows with non-temporal
// loads for a step of `batch` requests of at most max_len keys
// (pkv_load_policy).
bool stream_rows(const pkv_pool *p, int32_t batch, int32_t max_len) {
  if (p->load_policy == PKV_LOAD_STREAM) return true;
  if (p->load_policy == PKV_LOAD_CACHED) return false;
  // in double: no field combination can overflow the product
  const double row = (double)p->n_kv_heads * ((double)p->head_dim + v_dim(p)) *
                     (double)dtype_bytes(p->dtype);
  return batch == 1 && (double)p->n_layers * max_len * row > (double)kLastLevelCacheBytes;
}

// The table fields every gathering kernel takes.
template <class Args>
void set_table(Args &a, const pkv_pool *p) {
  a.req_to_token = p->req_to_token;
  a.max_ctx_len = p->max_ctx_len;
  a.page_shift = page_shift_of(p->page_size);
  a.table_stride = table_stride_of(p->max_ctx_len, a.page_shift);
}

// First byte of layer layer_id of a pool buffer whose rows are `dim` wide.
const char *layer_ptr(const void *buf, const pkv_pool *p, int32_t layer_id, int32_t dim) {
  const int64_t row = (int64_t)p->n_kv_heads * dim * (int64_t)dtype_bytes(p->dtype);
  return reinterpret_cast<const char *>(buf) + (int64_t)layer_id * p->size * row;
}
const char *k_layer_ptr(const pkv_pool *p, int32_t layer_id) {
  return layer_ptr(p->k_buffer, p, layer_id, p->head_dim);
}
const char *v_layer_ptr(const pkv_pool *p, int32_t layer_id) {
  return layer_ptr(p->v_buffer, p, layer_id, v_dim(p));
}

// Merge of split partials that skip_empty split kernels wrote: only the
// splits holding keys of each request are read (seq_lens, kv_start, chunk).
pkv::MergeArgs merge_args(const pkv::DecodeArgs &a, void *out, const int32_t *kv_start,
                          int32_t prefix_splits, int32_t prefix_chunk) {
  pkv::MergeArgs m{};
  m.o_part = a.o_part;
  m.ml_part = a.ml_part;
  m.out = out;
  m.rows = a.batch * a.n_heads;
  m.num_splits = a.num_splits;
  m.kv_start = kv_start;
  m.stride = a.split_stride;
  m.n_heads = a.n_heads;
  m.prefix_splits = prefix_splits;
  m.seq_lens = a.seq_lens;
  m.chunk = a.chunk;
  m.prefix_chunk = prefix_chunk > 0 ? prefix_chunk : 1;
  m.max_ctx_len = a.max_ctx_len;
  return m;
}

int32_t decode_chunk(int32_t max_len, int32_t num_splits) {
  int64_t c = ((int64_t)max_len + num_splits - 1) / num_splits;
  c = ((c + kSplitAlign - 1) / kSplitAlign) * kSplitAlign;
  return (int32_t)std::max<int64_t>(c, kSplitAlign);
}

}  // namespace

int pkv::note_hip_error(hipError_t e) {
  g_last_hip_error = (int32_t)e;
  return PKV_ERR_HIP;
}

extern "C" {

const char *pkv_status_string(pkv_status s) {
  switch (s) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "null pointer argument";
    case PKV_ERR_SHAPE: return "size, count or layer out of range";
    case PKV_ERR_DTYPE: return "unsupported dtype";
    case PKV_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case PKV_ERR_BAD_METADATA: return "inconsistent step metadata";
    case PKV_ERR_HIP: return "HIP runtime error";
    case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKV_ERR_SCRATCH_LIMIT: return "workspace needed exceeds the static scratch buffer";
  }
  return "unknown status";
}

int32_t pkv_last_hip_error(void) { return g_last_hip_error; }

pkv_status pkv_build_step(int32_t batch, const int32_t *req_pool_indices, const int32_t *seq_lens,
                          const int32_t *q_lens, const int32_t *req_to_token, int64_t num_reqs,
                          int64_t max_ctx_len, int32_t page_size, int32_t *kv_indptr,
                          int32_t *qo_indptr,
                          int32_t *out_cache_loc, int64_t out_cache_loc_cap, int64_t *n_new,
                          int32_t *max_len, int32_t *max_q_len, int32_t *prefill_order) {
  const int sh = page_shift_of(page_size);
  if (batch < 0 || sh < 0) return PKV_ERR_SHAPE;
  const int64_t stride = table_stride_of(max_ctx_len, sh);
  const int32_t off_mask = (1 << sh) - 1;
  if (!kv_indptr || !qo_indptr || !n_new || !max_len || !max_q_len) return PKV_ERR_NULL;
  if (batch > 0 && (!req_pool_indices || !seq_lens || !req_to_token)) return PKV_ERR_NULL;
  int64_t kv = 0, qo = 0;
  int32_t ml = 0, mq = 0;
  kv_indptr[0] = 0;
  qo_indptr[0] = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t r = req_pool_indices[b];
    const int32_t L = seq_lens[b];
    const int32_t ql = q_lens ? q_lens[b] : 1;
    if (r < 0 || r >= num_reqs || L < 1 || L > max_ctx_len || ql < 0 || ql > L)
      return PKV_ERR_BAD_METADATA;
    kv += L;
    if (kv > INT32_MAX) return PKV_ERR_BAD_METADATA;  // indptr entries are int32
    kv_indptr[b + 1] = (int32_t)kv;
    if (qo + ql > out_cache_loc_cap) return PKV_ERR_SHAPE;
    if (ql > 0 && !out_cache_loc) return PKV_ERR_NULL;
    const int32_t *row = req_to_token + r * stride;
    for (int32_t t = 0; t < ql; ++t) {
      const int32_t pos = L - ql + t;
      out_cache_loc[qo + t] = (int32_t)(((uint32_t)row[pos >> sh] << sh) | (uint32_t)(pos & off_mask));
    }
    qo += ql;
    qo_indptr[b + 1] = (int32_t)qo;
    ml = std::max(ml, L);
    mq = std::max(mq, ql);
  }
  *n_new = qo;
  *max_len = ml;
  *max_q_len = mq;
  if (prefill_order) {
    // longest context first; ties keep batch order
    for (int32_t b = 0; b < batch; ++b) prefill_order[b] = b;
    std::stable_sort(prefill_order, prefill_order + batch,
                     [&](int32_t x, int32_t y) { return seq_lens[x] > seq_lens[y]; });
  }
  return PKV_OK;
}

pkv_status pkv_build_positions(int32_t batch, const int32_t *seq_lens, const int32_t *q_lens,
                               int32_t *position_ids, int64_t capacity, int64_t *n_new) {
  if (batch < 0) return PKV_ERR_SHAPE;
  if (!n_new) return PKV_ERR_NULL;
  if (batch > 0 && !seq_lens) return PKV_ERR_NULL;
  int64_t qo = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t L = seq_lens[b];
    const int32_t ql = q_lens ? q_lens[b] : 1;
    if (ql < 0 || ql > L) return PKV_ERR_BAD_METADATA;
    if (qo + ql > capacity) return PKV_ERR_SHAPE;
    if (ql > 0 && !position_ids) return PKV_ERR_NULL;
    for (int32_t t = 0; t < ql; ++t) position_ids[qo + t] = L - ql + t;
    qo += ql;
  }
  *n_new = qo;
  return PKV_OK;
}

static_assert(PKV_PREFILL_BLOCK_ROWS == pkv::kPrefillBlockRows, "prefill block rows");

pkv_status pkv_prefill_blocks(int32_t batch, const int32_t *q_lens, const int32_t *order,
                              int32_t n_heads, int32_t n_kv_heads, int32_t *blocks,
                              int64_t capacity, int64_t *n_blocks) {
  if (batch < 0 || n_heads <= 0 || n_kv_heads <= 0 || n_heads % n_kv_heads != 0 ||
      capacity < 0)
    return PKV_ERR_SHAPE;
  if (!n_blocks) return PKV_ERR_NULL;
  if (batch > 0 && !q_lens) return PKV_ERR_NULL;
  const int64_t G = n_heads / n_kv_heads;
  std::vector<char> hit((size_t)batch, 0);
  int64_t n = 0;
  for (int32_t j = 0; j < batch; ++j) {
    const int32_t i = order ? order[j] : j;
    if (i < 0 || i >= batch || hit[(size_t)i]) return PKV_ERR_BAD_METADATA;
    hit[(size_t)i] = 1;
    if (q_lens[i] < 0) return PKV_ERR_SHAPE;
    const int64_t nblk = ((int64_t)q_lens[i] * G + pkv::kPrefillBlockRows - 1) /
                         pkv::kPrefillBlockRows;
    if (n + nblk > capacity) return PKV_ERR_SHAPE;
    if (nblk > 0 && !blocks) return PKV_ERR_NULL;
    for (int64_t x = 0; x < nblk; ++x, ++n) {  // last rows (most keys) first
      blocks[2 * n] = i;
      blocks[2 * n + 1] = (int32_t)(nblk - 1 - x);
    }
  }
  *n_blocks = n;
  return PKV_OK;
}

pkv_status pkv_validate_step(int64_t size, int64_t num_reqs, int64_t max_ctx_len,
                             int32_t page_size, const int32_t *req_to_token, int32_t batch,
                             const int32_t *req_pool_indices, const int32_t *seq_lens,
                             const int32_t *kv_indptr, const int32_t *qo_indptr,
                             const int32_t *out_cache_loc, int64_t n_new,
                             const int32_t *prefill_order) {
  const int sh = page_shift_of(page_size);
  if (batch < 0 || size <= 0 || num_reqs <= 0 || max_ctx_len <= 0) return PKV_ERR_SHAPE;
  if (sh < 0 || size % (int64_t(1) << sh) != 0) return PKV_ERR_SHAPE;
  const int64_t stride = table_stride_of(max_ctx_len, sh);
  const int64_t n_pages = size >> sh;
  const int32_t off_mask = (1 << sh) - 1;
  if (batch == 0) return n_new == 0 ? PKV_OK : PKV_ERR_BAD_METADATA;
  if (!req_to_token || !req_pool_indices || !seq_lens || !kv_indptr) return PKV_ERR_NULL;
  if (n_new > 0 && !out_cache_loc) return PKV_ERR_NULL;
  if (kv_indptr[0] != 0 || (qo_indptr && qo_indptr[0] != 0)) return PKV_ERR_BAD_METADATA;
  const int64_t expect_new = qo_indptr ? qo_indptr[batch] : batch;
  if (expect_new != n_new) return PKV_ERR_BAD_METADATA;
  std::unordered_set<int32_t> seen;
  seen.reserve((size_t)std::max<int64_t>(n_new, 0) * 2);
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t r = req_pool_indices[b];
    const int64_t L = seq_lens[b];
    if (r < 0 || r >= num_reqs || L < 1 || L > max_ctx_len) return PKV_ERR_BAD_METADATA;
    if ((int64_t)kv_indptr[b + 1] - kv_indptr[b] != L) return PKV_ERR_BAD_METADATA;
    const int64_t q0 = qo_indptr ? qo_indptr[b] : b;
    const int64_t ql = qo_indptr ? (int64_t)qo_indptr[b + 1] - qo_indptr[b] : 1;
    if (ql < 0 || ql > L || q0 + ql > n_new) return PKV_ERR_BAD_METADATA;
    const int32_t *row = req_to_token + r * stride;
    for (int64_t e = 0; e < ((L + off_mask) >> sh); ++e)  // entries of positions < L
      if (row[e] < 0 || row[e] >= n_pages) return PKV_ERR_BAD_METADATA;
    for (int64_t t = 0; t < ql; ++t) {
      const int32_t loc = out_cache_loc[q0 + t];
      if (loc < 0 || loc >= size) return PKV_ERR_BAD_METADATA;
      if (!seen.insert(loc).second) return PKV_ERR_BAD_METADATA;
      const int32_t pos = (int32_t)(L - ql + t);
      if (loc != (int32_t)(((uint32_t)row[pos >> sh] << sh) | (uint32_t)(pos & off_mask)))
        return PKV_ERR_BAD_METADATA;
    }
  }
  if (prefill_order) {
    std::vector<char> hit((size_t)batch, 0);
    for (int32_t b = 0; b < batch; ++b) {
      const int32_t x = prefill_order[b];
      if (x < 0 || x >= batch || hit[(size_t)x]) return PKV_ERR_BAD_METADATA;
      hit[(size_t)x] = 1;
    }
  }
  return PKV_OK;
}

pkv_status pkv_kv_store(const pkv_pool *pool, int32_t layer_id, const void *k_new,
                        const void *v_new, const int32_t *out_cache_loc, int64_t n_new,
                        void *stream) {
  pkv_status st = check_pool(pool, layer_id);
  if (st != PKV_OK) return st;
  if (n_new < 0) return PKV_ERR_SHAPE;
  if (n_new == 0) return PKV_OK;
  if (!k_new || !v_new || !out_cache_loc) return PKV_ERR_NULL;
  const int64_t row_bytes = (int64_t)pool->n_kv_heads * pool->head_dim * dtype_bytes(pool->dtype);
  const int64_t v_row_bytes = (int64_t)pool->n_kv_heads * v_dim(pool) * dtype_bytes(pool->dtype);
  if (row_bytes > INT32_MAX) return PKV_ERR_SHAPE;
  pkv::KvStoreArgs a{};
  a.k_layer = const_cast<char *>(k_layer_ptr(pool, layer_id));
  a.v_layer = const_cast<char *>(v_layer_ptr(pool, layer_id));
  a.k_new = k_new;
  a.v_new = v_new;
  a.out_cache_loc = out_cache_loc;
  a.n_new = n_new;
  a.size = pool->size;
  a.row_bytes = (int32_t)row_bytes;
  a.v_row_bytes = (int32_t)v_row_bytes;
  return hip_status(pkv::launch_kv_store(a, (hipStream_t)stream));
}

size_t pkv_decode_workspace_bytes(int32_t max_batch, int32_t n_heads, int32_t head_dim,
                                  int32_t num_splits) {
  if (max_batch <= 0 || n_heads <= 0 || head_dim <= 0 || num_splits <= 0) return 0;
  const size_t rows = (size_t)max_batch * n_heads * num_splits;
  const size_t o_bytes = rows * head_dim * sizeof(float);
  const size_t ml_bytes = rows * 2 * sizeof(float);
  return o_bytes + ml_bytes;
}

int32_t pkv_decode_pick_splits(int32_t batch, int32_t n_kv_heads, int32_t n_heads,
                               int32_t max_len, int64_t total_len, int32_t max_splits) {
  if (batch <= 0 || n_kv_heads <= 0 || n_heads <= 0 || max_len <= 0) return 1;
  max_splits = std::max(1, max_splits);
  if (total_len <= 0) total_len = (int64_t)batch * max_len;
  const int32_t group = std::max(1, n_heads / n_kv_heads);
  // head chunks per kv-head on the matrix-core path (16 query heads per wave)
  const int64_t chunks = (group + 15) / 16;
  // Wavefront-tokens of work: every (kv-head, head chunk) walks every token.
  const int64_t work = total_len * n_kv_heads * chunks;
  // Equal lengths: about 1024 long-running wavefronts (one per SIMD) keep the
  // per-split start-up and merge cost low.  Ragged lengths: splits of at most
  // 512 tokens, about 4K of them (four per SIMD), so that the device balances
  // the load; twice as many measured 2-3% slower on a 64-request batch (each
  // split pays the start-up chain again, and the merge reads more partials),
  // and much longer splits leave the end of the launch to a few of them.
  const bool ragged = (int64_t)batch * max_len > total_len + total_len / 4;
  int64_t chunk = ragged ? std::min<int64_t>(512, work / 4096)
                         : std::min<int64_t>(2048, work / 1024);
  chunk = std::max<int64_t>(chunk, 16);
  int64_t s = ((int64_t)max_len + chunk - 1) / chunk;
  // Ragged batches: the dispatcher deals workgroups to the 8 XCDs round-robin
  // in grid order (four kv-heads of one split, then the next split, then the
  // next request), so request b's split s starts on XCD (b * w + s * wgs) % 8
  // with w = wgs * num_splits workgroups per request.  When w is a multiple
  // of 8, split s of every request lands on the same XCDs, and the XCDs of
  // the low split indices, which every request has, get the most work.  An
  // odd split count makes w carry the fewest factors of 2 it can, spreading
  // the requests' splits over the most XCD offsets (with a multiple of 8
  // workgroups per split, every split already covers all XCDs alike).
  const int64_t wgs = (n_kv_heads * chunks + 3) / 4;  // workgroups per split
  if (ragged && batch > 1 && wgs % 8 != 0 && s % 2 == 0) ++s;
  s = std::min<int64_t>(s, max_splits);
  s = std::min<int64_t>(s, 65535);
  return (int32_t)std::max<int64_t>(1, s);
}

pkv_status pkv_paged_decode(const pkv_pool *pool, int32_t layer_id, const pkv_step *step,
                            const void *q, int32_t n_heads, float sm_scale, int32_t num_splits,
                            void *workspace, size_t ws_bytes, void *stream) {
  pkv_status st = check_pool(pool, layer_id);
  if (st != PKV_OK) return st;
  if (!step || !q || !workspace) return PKV_ERR_NULL;
  if (step->batch < 0 || n_heads <= 0 || n_heads % pool->n_kv_heads != 0 || num_splits <= 0 ||
      num_splits > 65535 || step->batch > 65535)
    return PKV_ERR_SHAPE;
  if (!dims_ok(pool)) return PKV_ERR_UNSUPPORTED;
  // unequal key / value widths run on the bf16 matrix-core kernel only
  if (pool->head_dim != v_dim(pool) && pool->dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (!std::isfinite(sm_scale)) return PKV_ERR_SHAPE;
  if (step->batch == 0) return PKV_OK;
  if (!step->req_pool_indices || !step->seq_lens) return PKV_ERR_NULL;
  if (step->max_len <= 0 || step->max_len > pool->max_ctx_len) return PKV_ERR_SHAPE;
  if (ws_bytes < pkv_decode_workspace_bytes(step->batch, n_heads, v_dim(pool), num_splits))
    return PKV_ERR_WORKSPACE_TOO_SMALL;
  const int32_t group = n_heads / pool->n_kv_heads;
  pkv::DecodeArgs a{};
  a.k_layer = k_layer_ptr(pool, layer_id);
  a.v_layer = v_layer_ptr(pool, layer_id);
  set_table(a, pool);
  a.req_pool_indices = step->req_pool_indices;
  a.seq_lens = step->seq_lens;
  a.q = q;
  a.o_part = reinterpret_cast<float *>(workspace);
  a.ml_part = a.o_part + (size_t)step->batch * n_heads * num_splits * v_dim(pool);
  a.batch = step->batch;
  a.n_heads = n_heads;
  a.n_kv_heads = pool->n_kv_heads;
  a.group = group;
  a.n_chunks = 0;
  a.heads_per_chunk = 0;
  a.num_splits = num_splits;
  a.chunk = decode_chunk(step->max_len, num_splits);
  a.kv_start = nullptr;
  a.split_stride = num_splits;
  a.skip_empty = 0;
  a.stream_rows = stream_rows(pool, step->batch, step->max_len);
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  return hip_status(pkv::launch_paged_decode(a, pool->dtype == PKV_BF16 ? 1 : 0,
                                              pool->head_dim, v_dim(pool), (hipStream_t)stream));
}

int32_t pkv_decode_load_kind(const pkv_pool *pool, int32_t batch, int32_t max_len) {
  if (!pool || batch < 0 || max_len < 0 || pool->n_layers <= 0 || pool->n_kv_heads <= 0 ||
      pool->head_dim <= 0 || pool->v_head_dim < 0 || !dtype_ok(pool->dtype) ||
      pool->load_policy < PKV_LOAD_AUTO || pool->load_policy > PKV_LOAD_STREAM)
    return -1;
  return stream_rows(pool, batch, max_len) ? 1 : 0;
}

int32_t pkv_decode_step_pick_splits(int32_t batch, int32_t n_kv_heads, int32_t n_heads,
                                    int32_t max_len, int64_t total_len, int32_t max_splits) {
  // Each split of the fused step is taken by a four-wave workgroup: a quarter
  // of the single-wave split count keeps the same work per wavefront.
  const int32_t s = pkv_decode_pick_splits(batch, n_kv_heads, n_heads, max_len, total_len, 65535);
  return std::max(1, std::min((s + 3) / 4, std::max(1, max_splits)));
}

pkv_status pkv_paged_decode_step(const pkv_pool *pool, int32_t layer_id, const pkv_step *step,
                                 const void *q, const void *k_new, const void *v_new,
                                 int32_t n_heads, float sm_scale, int32_t num_splits,
                                 void *workspace, size_t ws_bytes, int32_t *sync,
                                 int64_t sync_len, void *out, void *stream) {
  pkv_status st = check_pool(pool, layer_id);
  if (st != PKV_OK) return st;
  if (!step || !q || !workspace || !out || !sync) return PKV_ERR_NULL;
  if (step->batch < 0 || n_heads <= 0 || n_heads % pool->n_kv_heads != 0 || num_splits <= 0 ||
      num_splits > 65535 || step->batch > 65535)
    return PKV_ERR_SHAPE;
  if (!dims_ok(pool)) return PKV_ERR_UNSUPPORTED;
  if (!std::isfinite(sm_scale)) return PKV_ERR_SHAPE;
  if (step->batch == 0) return PKV_OK;
  if (!k_new || !v_new || !step->out_cache_loc || !step->req_pool_indices || !step->seq_lens)
    return PKV_ERR_NULL;
  if (step->n_new != step->batch) return PKV_ERR_SHAPE;  // one new token per request
  if (step->max_len <= 0 || step->max_len > pool->max_ctx_len) return PKV_ERR_SHAPE;
  if (sync_len < (int64_t)step->batch * n_heads) return PKV_ERR_SHAPE;
  if (ws_bytes < pkv_decode_workspace_bytes(step->batch, n_heads, v_dim(pool), num_splits))
    return PKV_ERR_WORKSPACE_TOO_SMALL;
  if (pool->dtype != PKV_BF16 || pool->head_dim != 128 || v_dim(pool) != 128) {
    // No fused kernel for this shape: the same step as three launches.
    st = pkv_kv_store(pool, layer_id, k_new, v_new, step->out_cache_loc, step->n_new, stream);
    if (st != PKV_OK) return st;
    st = pkv_paged_decode(pool, layer_id, step, q, n_heads, sm_scale, num_splits, workspace,
                          ws_bytes, stream);
    if (st != PKV_OK) return st;
    return pkv_paged_decode_merge(step->batch, n_heads, v_dim(pool), pool->dtype, num_splits,
                                  workspace, ws_bytes, out, stream);
  }
  pkv::StepArgs sa{};
  pkv::DecodeArgs &a = sa.d;
  a.k_layer = k_layer_ptr(pool, layer_id);
  a.v_layer = v_layer_ptr(pool, layer_id);
  set_table(a, pool);
  a.req_pool_indices = step->req_pool_indices;
  a.seq_lens = step->seq_lens;
  a.q = q;
  a.o_part = reinterpret_cast<float *>(workspace);
  a.ml_part = a.o_part + (size_t)step->batch * n_heads * num_splits * v_dim(pool);
  a.batch = step->batch;
  a.n_heads = n_heads;
  a.n_kv_heads = pool->n_kv_heads;
  a.group = n_heads / pool->n_kv_heads;
  a.n_chunks = 0;
  a.heads_per_chunk = 0;
  a.num_splits = num_splits;
  a.chunk = decode_chunk(step->max_len, num_splits);
  a.kv_start = nullptr;
  a.split_stride = num_splits;
  a.skip_empty = 0;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  sa.k_new = k_new;
  sa.v_new = v_new;
  sa.k_layer_w = const_cast<char *>(k_layer_ptr(pool, layer_id));
  sa.v_layer_w = const_cast<char *>(v_layer_ptr(pool, layer_id));
  sa.out_cache_loc = step->out_cache_loc;
  sa.sync = sync;
  sa.out = out;
  sa.tasks = 0;
  return hip_status(pkv::launch_decode_step(sa, (hipStream_t)stream));
}

pkv_status pkv_paged_decode_store(const pkv_pool *pool, int32_t layer_id, const pkv_step *step,
                                  const void *q, const void *k_new, const void *v_new,
                                  int32_t n_heads, float sm_scale, int32_t num_splits,
                                  void *workspace, size_t ws_bytes, void *out, void *stream) {
  pkv_status st = check_pool(pool, layer_id);
  if (st != PKV_OK) return st;
  if (!step || !q || !workspace || !out) return PKV_ERR_NULL;
  if (step->batch < 0 || n_heads <= 0 || n_heads % pool->n_kv_heads != 0 || num_splits <= 0 ||
      num_splits > 65535 || step->batch > 65535)
    return PKV_ERR_SHAPE;
  if (!dims_ok(pool)) return PKV_ERR_UNSUPPORTED;
  if (!std::isfinite(sm_scale)) return PKV_ERR_SHAPE;
  if (step->batch == 0) return PKV_OK;
  if (!k_new || !v_new || !step->out_cache_loc || !step->req_pool_indices || !step->seq_lens)
    return PKV_ERR_NULL;
  if (step->n_new != step->batch) return PKV_ERR_SHAPE;  // one new token per request
  if (step->max_len <= 0 || step->max_len > pool->max_ctx_len) return PKV_ERR_SHAPE;
  if (ws_bytes < pkv_decode_workspace_bytes(step->batch, n_heads, v_dim(pool), num_splits))
    return PKV_ERR_WORKSPACE_TOO_SMALL;
  if (!pkv::decode_mfma_shape(pool->dtype == PKV_BF16 ? 1 : 0, pool->head_dim, v_dim(pool))) {
    st = pkv_kv_store(pool, layer_id, k_new, v_new, step->out_cache_loc, step->n_new, stream);
    if (st != PKV_OK) return st;
    st = pkv_paged_decode(pool, layer_id, step, q, n_heads, sm_scale, num_splits, workspace,
                          ws_bytes, stream);
    if (st != PKV_OK) return st;
  } else {
    pkv::StepArgs sa{};
    pkv::DecodeArgs &a = sa.d;
    a.k_layer = k_layer_ptr(pool, layer_id);
    a.v_layer = v_layer_ptr(pool, layer_id);
    set_table(a, pool);
    a.req_pool_indices = step->req_pool_indices;
    a.seq_lens = step->seq_lens;
    a.q = q;
    a.o_part = reinterpret_cast<float *>(workspace);
    a.ml_part = a.o_part + (size_t)step->batch * n_heads * num_splits * v_dim(pool);
    a.batch = step->batch;
    a.n_heads = n_heads;
    a.n_kv_heads = pool->n_kv_heads;
    a.group = n_heads / pool->n_kv_heads;
    a.num_splits = num_splits;
    a.chunk = decode_chunk(step->max_len, num_splits);
    a.kv_start = nullptr;
    a.split_stride = num_splits;
    a.scale_log2 = sm_scale * 1.4426950408889634f;
    sa.k_new = k_new;
    sa.v_new = v_new;
    sa.k_layer_w = const_cast<char *>(k_layer_ptr(pool, layer_id));
    sa.v_layer_w = const_cast<char *>(v_layer_ptr(pool, layer_id));
    sa.out_cache_loc = step->out_cache_loc;
    // Splits past a request's keys leave no partial; the merge reads only the
    // ones that hold keys.
    a.skip_empty = 1;
    a.stream_rows = stream_rows(pool, step->batch, step->max_len);
    st = hip_status(pkv::launch_decode_split_store(sa, pool->head_dim, (hipStream_t)stream));
    if (st != PKV_OK) return st;
    pkv::MergeArgs m = merge_args(a, out, nullptr, 0, 0);
    return hip_status(pkv::launch_decode_merge(m, 1, v_dim(pool), (hipStream_t)stream));
  }
  return pkv_paged_decode_merge(step->batch, n_heads, v_dim(pool), pool->dtype, num_splits,
                                workspace, ws_bytes, out, stream);
}

pkv_status pkv_paged_decode_rope_store(const pkv_pool *pool, int32_t layer_id,
                                       const pkv_step *step, const void *q, const void *k_new,
                                       const void *v_new, const int32_t *position_ids,
                                       const float *freqs_cis, int64_t max_pos, int32_t n_heads,
                                       float sm_scale, int32_t num_splits, void *workspace,
                                       size_t ws_bytes, void *out, void *stream) {
  pkv_status st = check_pool(pool, layer_id);
  if (st != PKV_OK) return st;
  if (!step || !q || !workspace || !out) return PKV_ERR_NULL;
  if (step->batch < 0 || n_heads <= 0 || n_heads % pool->n_kv_heads != 0 || num_splits <= 0 ||
      num_splits > 65535 || step->batch > 65535 || max_pos <= 0)
    return PKV_ERR_SHAPE;
  if (!dims_ok(pool)) return PKV_ERR_UNSUPPORTED;
  if (pool->dtype != PKV_BF16 || pool->head_dim != 128 || v_dim(pool) != 128 ||
      n_heads / pool->n_kv_heads > 16)
    return PKV_ERR_UNSUPPORTED;
  if (!std::isfinite(sm_scale)) return PKV_ERR_SHAPE;
  if (step->batch == 0) return PKV_OK;
  if (!k_new || !v_new || !step->out_cache_loc || !step->req_pool_indices || !step->seq_lens ||
      !position_ids || !freqs_cis)
    return PKV_ERR_NULL;
  if (((uintptr_t)freqs_cis & 15u) != 0) return PKV_ERR_SHAPE;
  if (step->n_new != step->batch) return PKV_ERR_SHAPE;  // one new token per request
  if (step->max_len <= 0 || step->max_len > pool->max_ctx_len) return PKV_ERR_SHAPE;
  if (ws_bytes < pkv_decode_workspace_bytes(step->batch, n_heads, v_dim(pool), num_splits))
    return PKV_ERR_WORKSPACE_TOO_SMALL;
  pkv::StepArgs sa{};
  pkv::DecodeArgs &a = sa.d;
  a.k_layer = k_layer_ptr(pool, layer_id);
  a.v_layer = v_layer_ptr(pool, layer_id);
  set_table(a, pool);
  a.req_pool_indices = step->req_pool_indices;
  a.seq_lens = step->seq_lens;
  a.q = q;
  a.o_part = reinterpret_cast<float *>(workspace);
  a.ml_part = a.o_part + (size_t)step->batch * n_heads * num_splits * v_dim(pool);
  a.batch = step->batch;
  a.n_heads = n_heads;
  a.n_kv_heads = pool->n_kv_heads;
  a.group = n_heads / pool->n_kv_heads;
  a.num_splits = num_splits;
  a.chunk = decode_chunk(step->max_len, num_splits);
  a.kv_start = nullptr;
  a.split_stride = num_splits;
  a.skip_empty = 1;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  sa.k_new = k_new;
  sa.v_new = v_new;
  sa.k_layer_w = const_cast<char *>(k_layer_ptr(pool, layer_id));
  sa.v_layer_w = const_cast<char *>(v_layer_ptr(pool, layer_id));
  sa.out_cache_loc = step->out_cache_loc;
  sa.position_ids = position_ids;
  sa.freqs = freqs_cis;
  sa.max_pos = max_pos;
  a.stream_rows = stream_rows(pool, step->batch, step->max_len);
  st = hip_status(pkv::launch_decode_split_rope(sa, (hipStream_t)stream));
  if (st != PKV_OK) return st;
  pkv::MergeArgs m = merge_args(a, out, nullptr, 0, 0);
  return hip_status(pkv::launch_decode_merge(m, 1, v_dim(pool), (hipStream_t)stream));
}

pkv_status pkv_decode_prefix_groups(int32_t batch, const int32_t *req_pool_indices,
                                    const int32_t *seq_lens, const int32_t *req_to_token,
                                    int64_t num_reqs, int64_t max_ctx_len, int32_t page_size,
                                    int32_t min_prefix, int32_t *groups, int64_t groups_cap,
                                    int64_t *n_groups, int32_t *kv_start, int32_t *max_prefix,
                                    int32_t *max_members, int32_t *max_suffix) {
  const int sh = page_shift_of(page_size);
  if (batch < 0 || sh < 0 || groups_cap < 0) return PKV_ERR_SHAPE;
  if (!n_groups || !max_prefix || !max_members || !max_suffix) return PKV_ERR_NULL;
  if (batch > 0 && (!req_pool_indices || !seq_lens || !req_to_token || !kv_start))
    return PKV_ERR_NULL;
  if (groups_cap > 0 && !groups) return PKV_ERR_NULL;
  const int64_t stride = table_stride_of(max_ctx_len, sh);
  const int64_t ps = int64_t(1) << sh;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t r = req_pool_indices[b];
    if (r < 0 || r >= num_reqs || seq_lens[b] < 1 || seq_lens[b] > max_ctx_len)
      return PKV_ERR_BAD_METADATA;
    kv_start[b] = 0;
  }
  const int32_t min_p = std::max(1, min_prefix);
  auto row = [&](int32_t b) { return req_to_token + (int64_t)req_pool_indices[b] * stride; };
  // Positions both requests read through the same table entries (their
  // leading equal entries, in positions), leaving each request's last
  // position, the one this step writes, out of the shared range.
  auto shared = [&](int32_t x, int32_t y) -> int64_t {
    const int64_t cap = (int64_t)std::min(seq_lens[x], seq_lens[y]) - 1;
    const int32_t *rx = row(x), *ry = row(y);
    int64_t e = 0;
    while (e * ps < cap && rx[e] == ry[e]) ++e;
    return std::min(e * ps, cap);
  };
  // Requests whose first table entries agree, in batch order of the first.
  std::vector<std::vector<int32_t>> buckets;
  {
    std::vector<std::pair<int32_t, int32_t>> keyed;   // (first entry, b)
    for (int32_t b = 0; b < batch; ++b)
      if (seq_lens[b] >= 2) keyed.push_back({row(b)[0], b});
    std::stable_sort(keyed.begin(), keyed.end(),
                     [](const auto &u, const auto &v) { return u.first < v.first; });
    for (size_t i = 0; i < keyed.size();) {
      size_t j = i;
      std::vector<int32_t> mem;
      while (j < keyed.size() && keyed[j].first == keyed[i].first) mem.push_back(keyed[j++].second);
      if (mem.size() >= 2) buckets.push_back(mem);
      i = j;
    }
    std::sort(buckets.begin(), buckets.end(),
              [](const auto &u, const auto &v) { return u[0] < v[0]; });
  }
  int64_t ng = 0;
  int32_t mp = 0, mm = 0;
  for (auto &pending : buckets) {
    while (pending.size() >= 2) {
      // The lead is the longest pending request (earliest on ties): a
      // request's shared range ends before its own last position, so a short
      // lead would cut every member's.
      size_t li = 0;
      for (size_t i = 1; i < pending.size(); ++i)
        if (seq_lens[pending[i]] > seq_lens[pending[li]]) li = i;
      const int32_t lead = pending[li];
      std::vector<std::pair<int64_t, int32_t>> cand;   // (shared positions with lead, b)
      for (size_t i = 0; i < pending.size(); ++i)
        if (i != li) cand.push_back({shared(lead, pending[i]), pending[i]});
      std::stable_sort(cand.begin(), cand.end(),
                       [](const auto &u, const auto &v) { return u.first > v.first; });
      // Members = lead + the k-1 requests sharing the most with it; the
      // group's prefix is the smallest of their shared ranges.  Pick k for
      // the most positions read once instead of k times.
      int64_t best = 0;
      size_t best_k = 0;
      for (size_t k = 2; k <= std::min<size_t>(cand.size() + 1, PKV_PREFIX_GROUP_MAX); ++k) {
        const int64_t P = cand[k - 2].first;
        if (P < min_p) break;
        const int64_t gain = (int64_t)(k - 1) * P;
        if (gain > best) {
          best = gain;
          best_k = k;
        }
      }
      if (best_k == 0) {  // the lead shares too little with anyone: it stays alone
        pending.erase(pending.begin() + li);
        continue;
      }
      const int32_t P = (int32_t)cand[best_k - 2].first;
      if (ng >= groups_cap) return PKV_ERR_SHAPE;
      int32_t *rec = groups + ng * PKV_PREFIX_GROUP_INTS;
      for (int i = 0; i < PKV_PREFIX_GROUP_INTS; ++i) rec[i] = 0;
      rec[0] = P;
      rec[1] = (int32_t)best_k;
      rec[2] = lead;
      kv_start[lead] = P;
      std::vector<int32_t> taken{lead};
      for (size_t i = 0; i + 1 < best_k; ++i) {
        rec[3 + i] = cand[i].second;
        kv_start[cand[i].second] = P;
        taken.push_back(cand[i].second);
      }
      ++ng;
      mp = std::max(mp, P);
      mm = std::max(mm, (int32_t)best_k);
      std::vector<int32_t> rest;
      for (int32_t b : pending)
        if (std::find(taken.begin(), taken.end(), b) == taken.end()) rest.push_back(b);
      pending.swap(rest);
    }
  }
  int32_t msfx = 0;
  for (int32_t b = 0; b < batch; ++b) msfx = std::max(msfx, seq_lens[b] - kv_start[b]);
  *n_groups = ng;
  *max_prefix = mp;
  *max_members = mm;
  *max_suffix = msfx;
  return PKV_OK;
}

pkv_status pkv_paged_decode_shared(const pkv_pool *pool, int32_t layer_id, const pkv_step *step,
                                   const pkv_prefix_groups *pg, const void *q, const void *k_new,
                                   const void *v_new, int32_t n_heads, float sm_scale,
                                   int32_t num_splits, int32_t prefix_splits, void *workspace,
                                   size_t ws_bytes, void *out, void *stream) {
  pkv_status st = check_pool(pool, layer_id);
  if (st != PKV_OK) return st;
  if (!step || !q || !workspace || !out) return PKV_ERR_NULL;
  if (step->batch < 0 || n_heads <= 0 || n_heads % pool->n_kv_heads != 0 || num_splits <= 0 ||
      num_splits > 65535 || step->batch > 65535)
    return PKV_ERR_SHAPE;
  const bool mfma = pool->dtype == PKV_BF16 && pool->head_dim == 128 && v_dim(pool) == 128;
  if (!pg || pg->n_groups <= 0 || !mfma)  // nothing shared, or no matrix-core path: plain step
    return pkv_paged_decode_store(pool, layer_id, step, q, k_new, v_new, n_heads, sm_scale,
                                  num_splits, workspace, ws_bytes, out, stream);
  if (!std::isfinite(sm_scale)) return PKV_ERR_SHAPE;
  if (step->batch == 0) return PKV_OK;
  if (!k_new || !v_new || !step->out_cache_loc || !step->req_pool_indices || !step->seq_lens ||
      !pg->groups || !pg->kv_start)
    return PKV_ERR_NULL;
  if (step->n_new != step->batch) return PKV_ERR_SHAPE;
  if (prefix_splits <= 0 || prefix_splits > 65535 || pg->n_groups > 65535 ||
      pg->max_members < 1 || pg->max_members > PKV_PREFIX_GROUP_MAX || pg->max_prefix < 1 ||
      pg->max_suffix < 1 || pg->max_prefix > pool->max_ctx_len ||
      pg->max_suffix > pool->max_ctx_len || (int64_t)num_splits + prefix_splits > 65535)
    return PKV_ERR_SHAPE;
  const int32_t total = num_splits + prefix_splits;
  if (ws_bytes < pkv_decode_workspace_bytes(step->batch, n_heads, v_dim(pool), total))
    return PKV_ERR_WORKSPACE_TOO_SMALL;
  pkv::DecodeArgs a{};
  a.k_layer = k_layer_ptr(pool, layer_id);
  a.v_layer = v_layer_ptr(pool, layer_id);
  set_table(a, pool);
  a.req_pool_indices = step->req_pool_indices;
  a.seq_lens = step->seq_lens;
  a.q = q;
  a.o_part = reinterpret_cast<float *>(workspace);
  a.ml_part = a.o_part + (size_t)step->batch * n_heads * total * v_dim(pool);
  a.batch = step->batch;
  a.n_heads = n_heads;
  a.n_kv_heads = pool->n_kv_heads;
  a.group = n_heads / pool->n_kv_heads;
  a.num_splits = num_splits;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.split_stride = total;
  a.skip_empty = 1;
  // the groups' shared keys, once per group, and every request's own keys
  // from kv_start[b] with the new token's K/V write: one launch
  pkv::SharedArgs sh{};
  sh.pfx.d = a;
  sh.pfx.d.chunk = decode_chunk(pg->max_prefix, prefix_splits);
  sh.pfx.d.kv_start = nullptr;
  sh.pfx.groups = pg->groups;
  sh.pfx.n_groups = pg->n_groups;
  sh.pfx.prefix_splits = prefix_splits;
  sh.pfx.group_ints = PKV_PREFIX_GROUP_INTS;
  sh.pfx.max_members = pg->max_members;
  sh.sfx.d = a;
  sh.sfx.d.chunk = decode_chunk(pg->max_suffix, num_splits);
  sh.sfx.d.kv_start = pg->kv_start;
  sh.sfx.k_new = k_new;
  sh.sfx.v_new = v_new;
  sh.sfx.k_layer_w = const_cast<char *>(k_layer_ptr(pool, layer_id));
  sh.sfx.v_layer_w = const_cast<char *>(v_layer_ptr(pool, layer_id));
  sh.sfx.out_cache_loc = step->out_cache_loc;
  st = hip_status(pkv::launch_decode_shared(sh, (hipStream_t)stream));
  if (st != PKV_OK) return st;
  pkv::MergeArgs m = merge_args(sh.sfx.d, out, pg->kv_start, prefix_splits, sh.pfx.d.chunk);
  return hip_status(pkv::launch_decode_merge(m, 1, v_dim(pool), (hipStream_t)stream));
}

pkv_status pkv_decode_advance(const pkv_pool *pool, int32_t batch, const int32_t *req_pool_indices,
                              int32_t *seq_lens, int32_t *kv_indptr, int32_t *out_cache_loc,
                              int32_t *position_ids, void *stream) {
  pkv_status st = check_pool(pool, 0);
  if (st != PKV_OK) return st;
  if (batch < 0) return PKV_ERR_SHAPE;
  if (batch == 0) return PKV_OK;
  if (!req_pool_indices || !seq_lens || !out_cache_loc) return PKV_ERR_NULL;
  pkv::AdvanceArgs a{};
  set_table(a, pool);
  a.req_pool_indices = req_pool_indices;
  a.seq_lens = seq_lens;
  a.kv_indptr = kv_indptr;
  a.out_cache_loc = out_cache_loc;
  a.position_ids = position_ids;
  a.batch = batch;
  return hip_status(pkv::launch_decode_advance(a, (hipStream_t)stream));
}

}  // extern "C"

namespace {

pkv_status rope_store(const pkv_pool *pool, int32_t layer_id, const void *q, void *q_out,
                      int32_t n_heads, const void *k_new, const void *v_new,
                      const int32_t *position_ids, const float *freqs_cis, int64_t max_pos,
                      int32_t rope_dim, const int32_t *out_cache_loc, int64_t n_new,
                      void *stream) {
  pkv_status st = check_pool(pool, layer_id);
  if (st != PKV_OK) return st;
  if (n_new < 0 || max_pos <= 0 || n_heads <= 0 || n_heads % pool->n_kv_heads != 0)
    return PKV_ERR_SHAPE;
  if (!dims_ok(pool)) return PKV_ERR_UNSUPPORTED;
  // the rotated tail and the unrotated head of a row are whole 16-byte pieces
  const int32_t piece = pool->dtype == PKV_BF16 ? 8 : 4;
  if (rope_dim <= 0 || rope_dim > pool->head_dim || rope_dim % piece != 0) return PKV_ERR_SHAPE;
  if (n_new == 0) return PKV_OK;
  if (!q || !q_out || !k_new || !v_new || !position_ids || !freqs_cis || !out_cache_loc)
    return PKV_ERR_NULL;
  auto aligned = [](const void *p) { return ((uintptr_t)p & 15u) == 0; };
  if (!aligned(q) || !aligned(q_out) || !aligned(k_new) || !aligned(v_new) || !aligned(freqs_cis))
    return PKV_ERR_SHAPE;
  if (n_new > INT32_MAX) return PKV_ERR_SHAPE;
  pkv::RopeArgs a{};
  a.q = q;
  a.q_out = q_out;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_layer = const_cast<char *>(k_layer_ptr(pool, layer_id));
  a.v_layer = const_cast<char *>(v_layer_ptr(pool, layer_id));
  a.position_ids = position_ids;
  a.freqs = freqs_cis;
  a.max_pos = max_pos;
  a.out_cache_loc = out_cache_loc;
  a.n_new = n_new;
  a.n_heads = n_heads;
  a.n_kv_heads = pool->n_kv_heads;
  a.head_dim = pool->head_dim;
  a.v_head_dim = v_dim(pool);
  a.rope_dim = rope_dim;
  return hip_status(pkv::launch_rope_kv_store(a, pool->dtype == PKV_BF16 ? 1 : 0,
                                              (hipStream_t)stream));
}

}  // namespace

extern "C" {

pkv_status pkv_rope_kv_store(const pkv_pool *pool, int32_t layer_id, const void *q, void *q_out,
                             int32_t n_heads, const void *k_new, const void *v_new,
                             const int32_t *position_ids, const float *freqs_cis,
                             int64_t max_pos, const int32_t *out_cache_loc, int64_t n_new,
                             void *stream) {
  if (!pool) return PKV_ERR_NULL;
  return rope_store(pool, layer_id, q, q_out, n_heads, k_new, v_new, position_ids, freqs_cis,
                    max_pos, pool->head_dim, out_cache_loc, n_new, stream);
}

pkv_status pkv_rope_kv_store_partial(const pkv_pool *pool, int32_t layer_id, const void *q,
                                     void *q_out, int32_t n_heads, const void *k_new,
                                     const void *v_new, const int32_t *position_ids,
                                     const float *freqs_cis, int64_t max_pos, int32_t rope_dim,
                                     const int32_t *out_cache_loc, int64_t n_new, void *stream) {
  return rope_store(pool, layer_id, q, q_out, n_heads, k_new, v_new, position_ids, freqs_cis,
                    max_pos, rope_dim, out_cache_loc, n_new, stream);
}

pkv_status pkv_paged_decode_merge(int32_t batch, int32_t n_heads, int32_t head_dim,
                                  pkv_dtype out_dtype, int32_t num_splits, const void *workspace,
                                  size_t ws_bytes, void *out, void *stream) {
  if (!workspace || !out) return PKV_ERR_NULL;
  if (!dtype_ok(out_dtype)) return PKV_ERR_DTYPE;
  if (batch < 0 || n_heads <= 0 || num_splits <= 0) return PKV_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (batch == 0) return PKV_OK;
  if (ws_bytes < pkv_decode_workspace_bytes(batch, n_heads, head_dim, num_splits))
    return PKV_ERR_WORKSPACE_TOO_SMALL;
  pkv::MergeArgs a{};
  a.o_part = reinterpret_cast<const float *>(workspace);
  a.ml_part = a.o_part + (size_t)batch * n_heads * num_splits * head_dim;
  a.out = out;
  a.rows = batch * n_heads;
  a.num_splits = num_splits;
  a.kv_start = nullptr;
  a.stride = num_splits;
  a.n_heads = n_heads;
  a.prefix_splits = 0;
  return hip_status(pkv::launch_decode_merge(a, out_dtype == PKV_BF16 ? 1 : 0, head_dim,
                                             (hipStream_t)stream));
}

pkv_status pkv_paged_prefill(const pkv_pool *pool, int32_t layer_id, const pkv_step *step,
                             const void *q, int32_t n_heads, float sm_scale, int32_t causal,
                             void *out, void *stream) {
  pkv_status st = check_pool(pool, layer_id);
  if (st != PKV_OK) return st;
  if (pool->dtype != PKV_BF16) return PKV_ERR_DTYPE;
  if (!step || !q || !out) return PKV_ERR_NULL;
  if (step->batch < 0 || n_heads <= 0 || n_heads % pool->n_kv_heads != 0 || step->batch > 65535)
    return PKV_ERR_SHAPE;
  if (!dims_ok(pool)) return PKV_ERR_UNSUPPORTED;
  // the kernel ranks raw scores (the scale is applied in the exponent)
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.f)) return PKV_ERR_SHAPE;
  if (step->batch == 0 || step->n_new == 0) return PKV_OK;
  if (!step->req_pool_indices || !step->qo_indptr || !step->kv_indptr) return PKV_ERR_NULL;
  if (step->max_q_len <= 0 || step->max_q_len > pool->max_ctx_len) return PKV_ERR_SHAPE;
  pkv::PrefillArgs a{};
  a.k_layer = k_layer_ptr(pool, layer_id);
  a.v_layer = v_layer_ptr(pool, layer_id);
  set_table(a, pool);
  a.req_pool_indices = step->req_pool_indices;
  a.qo_indptr = step->qo_indptr;
  a.kv_indptr = step->kv_indptr;
  a.order = step->prefill_order;
  a.blocks = step->prefill_blocks;
  a.n_blocks = step->prefill_blocks ? step->n_prefill_blocks : 0;
  if (a.blocks && (a.n_blocks <= 0 || a.n_blocks * pool->n_kv_heads > INT32_MAX))
    return PKV_ERR_SHAPE;
  a.q = q;
  a.out = out;
  a.pool_size = pool->size;
  a.batch = step->batch;
  a.n_heads = n_heads;
  a.n_kv_heads = pool->n_kv_heads;
  a.group = n_heads / pool->n_kv_heads;
  a.max_q_len = step->max_q_len;
  a.causal = causal ? 1 : 0;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  return hip_status(pkv::launch_paged_prefill(a, pool->head_dim, v_dim(pool), (hipStream_t)stream));
}

}  // extern "C"

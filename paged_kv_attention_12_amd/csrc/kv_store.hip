// K/V write of one forward into the flat pool: row i of k_new / v_new goes to
// slot out_cache_loc[i] of the layer (AstrAI "Inference" guide, section
// "KVCache System", raw-index write; section "Attention Backend", the write
// precedes attention).  A bitwise copy: HBM-bound, 2 * n_new * row_bytes read
// and as much written.
#include "device.hpp"
#include "launch.hpp"

namespace pkv {

// One thread moves one W-byte piece of a K row and, where the value row is
// that wide (values may be narrower than keys), the same piece of the V row.
// Consecutive threads cover consecutive pieces of a row, so each row is read
// and written as one contiguous, fully coalesced run.
template <typename W>
__global__ void __launch_bounds__(256) kv_store_kernel(KvStoreArgs a, int64_t total_pieces,
                                                       int32_t pieces_per_row,
                                                       int32_t v_pieces_per_row) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total_pieces) return;
  const int64_t i = t / pieces_per_row;
  const int32_t c = (int32_t)(t - i * pieces_per_row);
  const int64_t loc = a.out_cache_loc[i];
  const W kx = reinterpret_cast<const W *>(a.k_new)[i * pieces_per_row + c];
  reinterpret_cast<W *>(a.k_layer)[loc * pieces_per_row + c] = kx;
  if (c < v_pieces_per_row) {
    const W vx = reinterpret_cast<const W *>(a.v_new)[i * v_pieces_per_row + c];
    reinterpret_cast<W *>(a.v_layer)[loc * v_pieces_per_row + c] = vx;
  }
}

hipError_t launch_kv_store(const KvStoreArgs &a, hipStream_t stream) {
  if (a.n_new == 0) return hipSuccess;
  const int threads = 256;
  auto go = [&](auto tag, int width) {
    using W = decltype(tag);
    const int32_t ppr = a.row_bytes / width;
    const int32_t vppr = a.v_row_bytes / width;
    const int64_t total = a.n_new * ppr;
    const int64_t blocks = (total + threads - 1) / threads;
    hipLaunchKernelGGL(kv_store_kernel<W>, dim3((uint32_t)blocks), dim3(threads), 0, stream, a,
                       total, ppr, vppr);
    return hipGetLastError();
  };
  const int32_t both = a.row_bytes | a.v_row_bytes;
  if (both % 16 == 0) return go(uint4{}, 16);
  if (both % 8 == 0) return go(uint2{}, 8);
  if (both % 4 == 0) return go(uint32_t{}, 4);
  return go(uint16_t{}, 2);
}

// Advance of a decode step's metadata to the next token, in place: every
// request grows by one token, its new token sits at position seq_len - 1 and
// is written to that position's slot; kv_indptr (the prefix sums of seq_lens)
// moves by b at entry b.  Positions past the table row are clamped (the
// caller keeps lengths within max_ctx_len; the clamp keeps reads in bounds).
__global__ void __launch_bounds__(256) decode_advance_kernel(const AdvanceArgs a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b > a.batch) return;
  if (b < a.batch) {
    const int32_t L = a.seq_lens[b] + 1;
    a.seq_lens[b] = L;
    if (a.position_ids) a.position_ids[b] = L - 1;
    const int64_t col = min((int64_t)L - 1, a.max_ctx_len - 1);
    a.out_cache_loc[b] = slot_of_pos(a.req_to_token + (int64_t)a.req_pool_indices[b] * a.table_stride,
                                     (uint32_t)col, a.page_shift);
  }
  if (a.kv_indptr) a.kv_indptr[b] += b;
}

hipError_t launch_decode_advance(const AdvanceArgs &a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  const int blocks = (a.batch + 1 + 255) / 256;
  hipLaunchKernelGGL(decode_advance_kernel, dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv

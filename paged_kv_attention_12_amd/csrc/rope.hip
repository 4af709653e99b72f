// Rotary embedding of one forward's new tokens fused with their K/V write
// (AstrAI "Inference" guide, section "Rotary Embedding Backend": a table of
// [cos, sin] pairs per position and dim pair, rows selected by position_ids,
// adjacent elements (2j, 2j+1) rotated as one complex number by cos + i sin;
// section "KV Cache": keys are rotated before they are written, so the cache
// holds rotated keys; section "KVCache System": the raw-index write
// buffer[layer, out_cache_loc] = k).
//
// HBM-bound: per new token the queries and keys are read and written once,
// the values copied, and each row reads its table row (d/2 [cos, sin] pairs,
// mostly from L2 since tokens of a step share few positions per row).
#include "device.hpp"
#include "launch.hpp"

namespace pkv {

namespace {

template <typename T>
struct Piece;

// bf16: a 16-byte piece is 8 elements, 4 pairs.
template <>
struct Piece<uint16_t> {
  static constexpr int E = 8;
  __device__ static void load(const uint4 &w, float (&x)[E]) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = bf16_lo(u[k]);
      x[2 * k + 1] = bf16_hi(u[k]);
    }
  }
  __device__ static uint4 store(const float (&x)[E]) {
    return make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                      pack_bf16x2(x[6], x[7]));
  }
};

// fp32: a 16-byte piece is 4 elements, 2 pairs.
template <>
struct Piece<float> {
  static constexpr int E = 4;
  __device__ static void load(const uint4 &w, float (&x)[E]) {
    x[0] = __uint_as_float(w.x);
    x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z);
    x[3] = __uint_as_float(w.w);
  }
  __device__ static uint4 store(const float (&x)[E]) {
    return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                      __float_as_uint(x[3]));
  }
};

// Pair (a, b) of the piece times (c + i s): (a c - b s, a s + b c), in fp32.
template <typename T>
__device__ __forceinline__ uint4 rotate(const uint4 &w, const float *f) {
  constexpr int E = Piece<T>::E;
  float x[E], cs[E];
#pragma unroll
  for (int k = 0; k < E; k += 4) {
    const float4 v = *reinterpret_cast<const float4 *>(f + k);
    cs[k] = v.x;
    cs[k + 1] = v.y;
    cs[k + 2] = v.z;
    cs[k + 3] = v.w;
  }
  Piece<T>::load(w, x);
  float y[E];
#pragma unroll
  for (int j = 0; j < E / 2; ++j) {
    const float a = x[2 * j], b = x[2 * j + 1];
    const float c = cs[2 * j], s = cs[2 * j + 1];
    y[2 * j] = fmaf(a, c, -(b * s));
    y[2 * j + 1] = fmaf(a, s, b * c);
  }
  return Piece<T>::store(y);
}

// One thread per 16-byte piece.  Threads [0, q_pieces) handle query pieces
// (token i, head h, piece c in row order); the next kv_pieces threads each
// handle one key piece, written to the pool, and the matching value piece
// where the value row is that wide.  Pieces in the last rope_dim dims of a
// row are rotated (table entry (c * E - (head_dim - rope_dim)) / 2 onwards);
// the others are copied unchanged (MLA rows: only the qk_rope part turns).
// Consecutive threads cover consecutive pieces of a row, so every row is one
// coalesced run.  Positions outside [0, max_pos) read the nearest table row
// (the caller guarantees valid positions; the clamp only keeps reads in
// bounds).  q, k_new and v_new are read once, with non-temporal loads, so
// that they do not displace the table rows every head row of a token reads
// (4% faster on a 20356-token step than cached loads; non-temporal stores
// measured no faster).
template <typename T>
__global__ void __launch_bounds__(256) rope_kv_store_kernel(const RopeArgs a, int64_t q_pieces,
                                                            int64_t kv_pieces) {
  constexpr int E = Piece<T>::E;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int ppr = a.head_dim / E;      // pieces per query / key row
  const int vppr = a.v_head_dim / E;   // pieces per value row
  const int first_rot = (a.head_dim - a.rope_dim) / E;  // first rotated piece
  if (t < q_pieces) {
    const int64_t row = t / ppr;
    const int c = (int)(t - row * ppr);
    const uint4 w = load16_nt(reinterpret_cast<const uint4 *>(a.q) + t);
    uint4 r = w;
    if (c >= first_rot) {
      const int64_t i = row / a.n_heads;
      const int64_t p = min(max((int64_t)a.position_ids[i], (int64_t)0), a.max_pos - 1);
      r = rotate<T>(w, a.freqs + p * a.rope_dim + (int64_t)(c - first_rot) * E);
    }
    reinterpret_cast<uint4 *>(a.q_out)[t] = r;
  } else if (t < q_pieces + kv_pieces) {
    const int64_t u = t - q_pieces;
    const int64_t row = u / ppr;
    const int c = (int)(u - row * ppr);
    const int64_t i = row / a.n_kv_heads;
    const int64_t hk = row - i * a.n_kv_heads;
    const int64_t loc = a.out_cache_loc[i];
    const uint4 kw = load16_nt(reinterpret_cast<const uint4 *>(a.k_new) + u);
    uint4 kr = kw;
    if (c >= first_rot) {
      const int64_t p = min(max((int64_t)a.position_ids[i], (int64_t)0), a.max_pos - 1);
      kr = rotate<T>(kw, a.freqs + p * a.rope_dim + (int64_t)(c - first_rot) * E);
    }
    reinterpret_cast<uint4 *>(a.k_layer)[(loc * a.n_kv_heads + hk) * ppr + c] = kr;
    if (c < vppr) {
      const uint4 vw = load16_nt(reinterpret_cast<const uint4 *>(a.v_new) + row * vppr + c);
      reinterpret_cast<uint4 *>(a.v_layer)[(loc * a.n_kv_heads + hk) * vppr + c] = vw;
    }
  }
}

}  // namespace

hipError_t launch_rope_kv_store(const RopeArgs &a, int dtype, hipStream_t stream) {
  if (a.n_new == 0) return hipSuccess;
  const int E = dtype == 1 ? 8 : 4;
  const int64_t ppr = a.head_dim / E;
  const int64_t q_pieces = a.n_new * a.n_heads * ppr;
  const int64_t kv_pieces = a.n_new * a.n_kv_heads * ppr;
  const int64_t blocks = (q_pieces + kv_pieces + 255) / 256;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (dtype == 1)
    hipLaunchKernelGGL(rope_kv_store_kernel<uint16_t>, dim3((uint32_t)blocks), dim3(256), 0, stream,
                       a, q_pieces, kv_pieces);
  else
    hipLaunchKernelGGL(rope_kv_store_kernel<float>, dim3((uint32_t)blocks), dim3(256), 0, stream, a,
                       q_pieces, kv_pieces);
  return hipGetLastError();
}

}  // namespace pkv

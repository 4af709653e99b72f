// Split-KV paged decode and the merge of its partials.
//
// What is computed (AstrAI "Inference" guide, section "KV Cache"): for every
// request b and query head h, o = sum_j softmax_j(q . k_j * sm_scale) v_j over
// the request's seq_lens[b] cached keys of kv-head h / G, which the kernel
// gathers itself through req_to_token (section "Attention Backend": one-token
// pages, no separate gather).  The key range is cut into num_splits logical
// splits; each split leaves a partial (m, l, o) in a caller-owned workspace
// and a merge pass combines them (commit history of
// tests/inference/test_cache.py, entries on the split-partial workspace).
//
// Mapping on CDNA4.  One wavefront owns one (request, split, kv-head, chunk of
// <= 8 query heads of that kv-head's group).  A K or V row of one kv-head is
// head_dim * sizeof(T) contiguous bytes (256 B for bf16, d = 128); LPT lanes
// cover it with one 16-byte load each, so a wave gathers TPW = 64 / LPT whole
// rows per load instruction and every row is one coalesced run.  Each lane
// keeps its 16-byte slice of the chunk's query heads in registers; the partial
// dot products are summed across the LPT lanes of a row with DPP (no LDS), and
// every row group keeps its own online-softmax state (m, l, acc) in base 2,
// so the inner loop needs no cross-row traffic.  The TPW row states are
// combined once at the end.  The four waves of a workgroup handle four
// consecutive (kv-head, chunk) tasks of the same (request, split), so the
// slot's kv-head rows that sit next to each other in HBM are fetched together.
#include <math.h>

#include "device.hpp"
#include "launch.hpp"

namespace pkv {

namespace {

constexpr float kNegInf = -INFINITY;

template <typename T>
__device__ __forceinline__ float elem(const uint4 &w, int e) {
  const uint32_t x[4] = {w.x, w.y, w.z, w.w};
  if constexpr (sizeof(T) == 2) {
    return (e & 1) ? bf16_hi(x[e >> 1]) : bf16_lo(x[e >> 1]);
  } else {
    return __uint_as_float(x[e]);
  }
}

// Partial dot product of a lane's 16-byte slices of q and k.
template <typename T>
__device__ __forceinline__ float slice_dot(const uint4 &q, const uint4 &k) {
  if constexpr (sizeof(T) == 2) {
    float s = dot2_bf16(q.x, k.x, 0.f);
    s = dot2_bf16(q.y, k.y, s);
    s = dot2_bf16(q.z, k.z, s);
    return dot2_bf16(q.w, k.w, s);
  } else {
    float s = __uint_as_float(q.x) * __uint_as_float(k.x);
    s = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), s);
    s = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), s);
    return fmaf(__uint_as_float(q.w), __uint_as_float(k.w), s);
  }
}

template <typename T, int D, int NG, int U>
__global__ void __launch_bounds__(256) decode_split_kernel(const DecodeArgs a) {
  constexpr int EPL = 16 / (int)sizeof(T);  // elements per lane per row
  constexpr int LPT = D / EPL;              // lanes per row
  constexpr int TPW = 64 / LPT;             // rows per wave per load
  constexpr int STEP = TPW * U;             // tokens per iteration
  static_assert(LPT >= 4 && LPT <= 64 && 64 % LPT == 0, "row width");

  const int lane = threadIdx.x & 63;
  const int task = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (task >= a.n_kv_heads * a.n_chunks) return;
  const int b = blockIdx.z;
  const int s = blockIdx.y;
  const int hk = task / a.n_chunks;
  const int g0 = (task - hk * a.n_chunks) * a.heads_per_chunk;
  const int ng = min(a.heads_per_chunk, a.group - g0);
  const int h0 = hk * a.group + g0;
  const int row = lane / LPT;
  const int part = lane - row * LPT;
  const int S = a.num_splits;

  const int L = a.seq_lens[b];
  const int start = s * a.chunk;
  const int end = min(L, start + a.chunk);
  const int64_t p0 = ((int64_t)b * a.n_heads + h0) * S + s;  // partial row of head h0

  if (start >= end) {  // empty split: (m, l) = (-inf, 0), o = 0
    if (row == 0) {
      for (int g = 0; g < ng; ++g) {
        float *o = a.o_part + (p0 + (int64_t)g * S) * D + part * EPL;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] = 0.f;
        if (part == 0) {
          a.ml_part[(p0 + (int64_t)g * S) * 2 + 0] = kNegInf;
          a.ml_part[(p0 + (int64_t)g * S) * 2 + 1] = 0.f;
        }
      }
    }
    return;
  }

  uint4 qv[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    qv[g] = make_uint4(0u, 0u, 0u, 0u);
    if (g < ng)
      qv[g] = load16(reinterpret_cast<const T *>(a.q) +
                     ((int64_t)b * a.n_heads + h0 + g) * D + part * EPL);
  }

  const int32_t *table = a.req_to_token + (int64_t)a.req_pool_indices[b] * a.max_ctx_len;
  const int64_t row_elems = (int64_t)a.n_kv_heads * D;
  const T *kbase = reinterpret_cast<const T *>(a.k_layer) + (int64_t)hk * D + part * EPL;
  const T *vbase = reinterpret_cast<const T *>(a.v_layer) + (int64_t)hk * D + part * EPL;

  float m[NG], l[NG], acc[NG][EPL];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  for (int j0 = start; j0 < end; j0 += STEP) {
    int slot[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * TPW + row;
      ok[u] = j < end;
      slot[u] = ok[u] ? table[j] : 0;
    }
    uint4 kx[U], vx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      kx[u] = make_uint4(0u, 0u, 0u, 0u);
      vx[u] = make_uint4(0u, 0u, 0u, 0u);
      if (ok[u]) {
        kx[u] = load16(kbase + (int64_t)slot[u] * row_elems);
        vx[u] = load16(vbase + (int64_t)slot[u] * row_elems);
      }
    }
    float sc[U][NG];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int g = 0; g < NG; ++g) sc[u][g] = group_sum<LPT>(slice_dot<T>(qv[g], kx[u]));

#pragma unroll
    for (int g = 0; g < NG; ++g) {
      float mt = kNegInf;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        sc[u][g] = ok[u] ? sc[u][g] * a.scale_log2 : kNegInf;
        mt = fmaxf(mt, sc[u][g]);
      }
      const float mn = fmaxf(m[g], mt);
      const float mref = (mn == kNegInf) ? 0.f : mn;
      const float alpha = fast_exp2(m[g] - mref);
      l[g] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = fast_exp2(sc[u][g] - mref);
        l[g] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(p, elem<T>(vx[u], e), acc[g][e]);
      }
      m[g] = mn;
    }
  }

  // Combine the TPW row states of the wave (rows sit LPT lanes apart).
#pragma unroll
  for (int X = LPT; X < 64; X <<= 1) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const float mo = __shfl_xor(m[g], X);
      const float lo = __shfl_xor(l[g], X);
      const float M = fmaxf(m[g], mo);
      const float Mr = (M == kNegInf) ? 0.f : M;
      const float ca = fast_exp2(m[g] - Mr);
      const float cb = fast_exp2(mo - Mr);
      l[g] = l[g] * ca + lo * cb;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] = acc[g][e] * ca + __shfl_xor(acc[g][e], X) * cb;
      m[g] = M;
    }
  }

  if (row == 0) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g < ng) {
        const int64_t pr = p0 + (int64_t)g * S;
        const float inv = 1.f / l[g];
        float4 *o = reinterpret_cast<float4 *>(a.o_part + pr * D + part * EPL);
#pragma unroll
        for (int e = 0; e < EPL; e += 4)
          o[e / 4] = make_float4(acc[g][e] * inv, acc[g][e + 1] * inv, acc[g][e + 2] * inv,
                                 acc[g][e + 3] * inv);
        if (part == 0) {
          a.ml_part[pr * 2 + 0] = m[g];
          a.ml_part[pr * 2 + 1] = l[g];
        }
      }
    }
  }
}

// One group of D/4 threads per (request, head) row; 4 consecutive dims each.
template <typename T, int D>
__global__ void __launch_bounds__(256) decode_merge_kernel(const MergeArgs a) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const int r = blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  if (r >= a.rows) return;
  const int S = a.num_splits;
  const float *ml = a.ml_part + (int64_t)r * S * 2;
  const float *op = a.o_part + (int64_t)r * S * D + c * 4;
  float M = kNegInf;
  for (int s = 0; s < S; ++s)
    if (ml[2 * s + 1] > 0.f) M = fmaxf(M, ml[2 * s]);
  float den = 0.f, n0 = 0.f, n1 = 0.f, n2 = 0.f, n3 = 0.f;
  for (int s = 0; s < S; ++s) {
    const float ls = ml[2 * s + 1];
    if (ls > 0.f) {
      const float w = ls * fast_exp2(ml[2 * s] - M);
      const float4 o = *reinterpret_cast<const float4 *>(op + (int64_t)s * D);
      den += w;
      n0 = fmaf(w, o.x, n0);
      n1 = fmaf(w, o.y, n1);
      n2 = fmaf(w, o.z, n2);
      n3 = fmaf(w, o.w, n3);
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  if constexpr (sizeof(T) == 2) {
    uint2 w;
    w.x = pack_bf16x2(n0 * inv, n1 * inv);
    w.y = pack_bf16x2(n2 * inv, n3 * inv);
    *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(a.out) + (int64_t)r * D + c * 4) = w;
  } else {
    *reinterpret_cast<float4 *>(reinterpret_cast<float *>(a.out) + (int64_t)r * D + c * 4) =
        make_float4(n0 * inv, n1 * inv, n2 * inv, n3 * inv);
  }
}

template <typename T, int D>
hipError_t decode_dispatch_ng(const DecodeArgs &a, hipStream_t stream) {
  const dim3 grid((a.n_kv_heads * a.n_chunks + 3) / 4, a.num_splits, a.batch);
  const dim3 block(256);
#define PKV_NG_CASE(NGV, UV)                                                              \
  case NGV:                                                                               \
    hipLaunchKernelGGL((decode_split_kernel<T, D, NGV, UV>), grid, block, 0, stream, a); \
    break;
  switch (a.heads_per_chunk) {
    PKV_NG_CASE(1, 4)
    PKV_NG_CASE(2, 4)
    PKV_NG_CASE(3, 4)
    PKV_NG_CASE(4, 4)
    PKV_NG_CASE(5, 2)
    PKV_NG_CASE(6, 2)
    PKV_NG_CASE(7, 2)
    PKV_NG_CASE(8, 2)
    default:
      return hipErrorInvalidValue;
  }
#undef PKV_NG_CASE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_paged_decode(const DecodeArgs &a, int dtype, int head_dim, hipStream_t stream) {
  if (dtype == 1) {
    if (head_dim == 128) return decode_dispatch_ng<uint16_t, 128>(a, stream);
    if (head_dim == 64) return decode_dispatch_ng<uint16_t, 64>(a, stream);
  } else {
    if (head_dim == 128) return decode_dispatch_ng<float, 128>(a, stream);
    if (head_dim == 64) return decode_dispatch_ng<float, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_merge(const MergeArgs &a, int dtype, int head_dim, hipStream_t stream) {
  const int tpr = head_dim / 4;
  const int rpb = 256 / tpr;
  const dim3 grid((a.rows + rpb - 1) / rpb);
  if (dtype == 1) {
    if (head_dim == 128)
      hipLaunchKernelGGL((decode_merge_kernel<uint16_t, 128>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_merge_kernel<uint16_t, 64>), grid, dim3(256), 0, stream, a);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((decode_merge_kernel<float, 128>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_merge_kernel<float, 64>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace pkv

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

// Slot ids of one split are staged in LDS in rounds of this many tokens.
constexpr int kSlotTile = 2048;

// Keys of split s: [s * chunk, min(L, (s + 1) * chunk)), except that the last
// split also takes every key past num_splits * chunk, so a request that has
// grown past the host max_len the split size came from (a replayed graph
// whose lengths advance on the device) is still attended whole, only more
// slowly.  A length past max_ctx_len cannot be addressed through the table;
// such a request attends nothing and its partials are NaN (split_overrun), so
// the merged output is NaN instead of silently wrong.
__device__ __forceinline__ bool split_overrun(const DecodeArgs &a, int L) {
  return L > a.max_ctx_len;
}
__device__ __forceinline__ int split_end(const DecodeArgs &a, int s, int start, int L) {
  if (split_overrun(a, L)) return start;
  return s == a.num_splits - 1 ? L : min(L, start + a.chunk);
}

template <typename T, int D, int NG, int U>
__global__ void __launch_bounds__(256) decode_split_kernel(const DecodeArgs a) {
  constexpr int EPL = 16 / (int)sizeof(T);  // elements per lane per row
  constexpr int LPT = D / EPL;              // lanes per row
  constexpr int TPW = 64 / LPT;             // rows per wave per load
  constexpr int STEP = TPW * U;             // tokens per iteration
  static_assert(LPT >= 4 && LPT <= 64 && 64 % LPT == 0, "row width");
  __shared__ int32_t s_slot[kSlotTile];

  const int b = blockIdx.z;
  const int s = blockIdx.y;
  const int L = a.seq_lens[b];
  const int pool_row = a.req_pool_indices[b];
  const int start = s * a.chunk;
  const int end = split_end(a, s, start, L);

  const int lane = threadIdx.x & 63;
  const int task = blockIdx.x * 4 + (threadIdx.x >> 6);
  // Waves past the last task still take part in the workgroup barriers.
  const bool active = task < a.n_kv_heads * a.n_chunks;
  const int hk = active ? task / a.n_chunks : 0;
  const int g0 = active ? (task - hk * a.n_chunks) * a.heads_per_chunk : 0;
  const int ng = active ? min(a.heads_per_chunk, a.group - g0) : 0;
  const int h0 = hk * a.group + g0;
  const int row = lane / LPT;
  const int part = lane - row * LPT;
  const int S = a.num_splits;
  const int64_t p0 = ((int64_t)b * a.n_heads + h0) * S + s;  // partial row of head h0

  if (start >= end) {  // empty split (uniform over the workgroup): (-inf, 0), o = 0
    const bool bad = split_overrun(a, L);
    const float ov = bad ? NAN : 0.f;
    if (active && row == 0) {
      for (int g = 0; g < ng; ++g) {
        float4 *o = reinterpret_cast<float4 *>(a.o_part + (p0 + (int64_t)g * S) * D + part * EPL);
#pragma unroll
        for (int e = 0; e < EPL; e += 4) o[e / 4] = make_float4(ov, ov, ov, ov);
        if (part == 0) {
          a.ml_part[(p0 + (int64_t)g * S) * 2 + 0] = bad ? NAN : kNegInf;
          a.ml_part[(p0 + (int64_t)g * S) * 2 + 1] = bad ? 1.f : 0.f;
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

  const int32_t *table = a.req_to_token + (int64_t)pool_row * a.table_stride;
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

  // Gather the rows of tokens j0 + u * TPW + row (u < U) of the current round.
  auto fetch = [&](uint4(&kx)[U], uint4(&vx)[U], int j0, int r0, int r1) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * TPW + row;
      kx[u] = make_uint4(0u, 0u, 0u, 0u);
      vx[u] = make_uint4(0u, 0u, 0u, 0u);
      if (j < r1) {
        const int64_t off = (int64_t)s_slot[j - r0] * row_elems;
        kx[u] = load16(kbase + off);
        vx[u] = load16(vbase + off);
      }
    }
  };

  // Scores, then the online-softmax update of this row group's state.
  auto process = [&](const uint4(&kx)[U], const uint4(&vx)[U], int j0, int r1) {
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
        const bool ok = j0 + u * TPW + row < r1;
        sc[u][g] = ok ? sc[u][g] * a.scale_log2 : kNegInf;
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
  };

  uint4 ka[U], va[U], kb[U], vb[U];
  for (int r0 = start; r0 < end; r0 += kSlotTile) {
    const int r1 = min(end, r0 + kSlotTile);
    if (r0 != start) __syncthreads();  // every wave is done with the previous round
    for (int j = r0 + (int)threadIdx.x; j < r1; j += 256)
      s_slot[j - r0] = slot_of_pos(table, (uint32_t)j, a.page_shift);
    __syncthreads();
    if (!active) continue;
    // Two register sets: the rows of the next iteration are in flight while
    // the current ones are used.
    int j0 = r0;
    fetch(ka, va, j0, r0, r1);
    while (true) {
      const int j1 = j0 + STEP;
      if (j1 < r1) fetch(kb, vb, j1, r0, r1);
      process(ka, va, j0, r1);
      if (j1 >= r1) break;
      const int j2 = j1 + STEP;
      if (j2 < r1) fetch(ka, va, j2, r0, r1);
      process(kb, vb, j1, r1);
      if (j2 >= r1) break;
      j0 = j2;
    }
  }
  if (!active) return;

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

// One workgroup of NT threads per (request, head) row.  The splits are
// spread over NT / (D/4) split groups of D/4 threads (4 dims each).  Each
// thread loads (m, l, o) of up to KB splits in one batch, the row maximum is
// reduced over the workgroup, then every thread weighs what it holds: one
// memory round trip for up to SG * KB splits.  Group sums are added through
// LDS.
template <typename T, int D, int KB, int NT>
__global__ void __launch_bounds__(NT) decode_merge_kernel(const MergeArgs a) {
  constexpr int TPR = D / 4;
  constexpr int SG = NT / TPR;
  constexpr int NW = NT / 64;  // wavefronts
  static_assert(NT % 64 == 0 && SG >= 1, "workgroup shape");
  __shared__ float s_red[NW];
  __shared__ float4 s_num[SG][TPR];
  __shared__ float s_den[SG];
  const int r = blockIdx.x;
  const int t = threadIdx.x;
  // Splits of this row (rows are a.stride splits apart).  Without seq_lens:
  // all num_splits (empty ones hold weight-0 partials).  With seq_lens, only
  // the splits that hold keys were written: own split s covers keys from
  // kv_start + s * chunk (the last one any excess), prefix split s keys from
  // s * prefix_chunk below P = kv_start; those partials sit after the own
  // num_splits in the row, so both are read as one run with a gap skipped.
  int S = a.num_splits, n_own = a.num_splits;
  if (a.seq_lens) {
    const int b = r / a.n_heads;
    const int base = a.kv_start ? a.kv_start[b] : 0;
    const int len = a.seq_lens[b] - base;
    n_own = len <= 0 ? 0 : min(a.num_splits, (len + a.chunk - 1) / a.chunk);
    if (a.seq_lens[b] > a.max_ctx_len) n_own = a.num_splits;  // NaN partials, all written
    const int n_pfx = base > 0 ? min(a.prefix_splits, (base + a.prefix_chunk - 1) / a.prefix_chunk)
                               : 0;
    S = n_own + n_pfx;
  } else if (a.kv_start && a.kv_start[r / a.n_heads] > 0) {
    S = a.num_splits + a.prefix_splits;
    n_own = S;
  }
  // slot of the k-th split read: own splits first, then the prefix ones
  const int gap = a.num_splits - n_own;
  const int sg = t / TPR;
  const int c = t - sg * TPR;
  const float *ml = a.ml_part + (int64_t)r * a.stride * 2;
  const float *op = a.o_part + (int64_t)r * a.stride * D + c * 4;

  float den = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  float M = kNegInf;  // running maximum over the batches seen so far
  // Every thread runs every batch (the batch holds the workgroup barriers);
  // split groups past the last split carry weight 0.
  for (int base = 0; base < S; base += SG * KB) {
    const int s0 = base + sg;
    float4 ov[KB];
    float mv[KB], lv[KB];
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int sk = min(s0 + SG * k, S - 1);
      const int s = sk < n_own ? sk : sk + gap;
      ov[k] = *reinterpret_cast<const float4 *>(op + (int64_t)s * D);
      mv[k] = ml[2 * s];
      lv[k] = (s0 + SG * k < S) ? ml[2 * s + 1] : 0.f;
    }
    // maximum over this batch's non-empty splits, across the workgroup
    float bm = M;
#pragma unroll
    for (int k = 0; k < KB; ++k)
      if (lv[k] > 0.f) bm = fmaxf(bm, mv[k]);
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) bm = fmaxf(bm, __shfl_xor(bm, x));
    __syncthreads();  // s_red of the previous batch has been read
    if ((t & 63) == 0) s_red[t >> 6] = bm;
    __syncthreads();
    float Mn = s_red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) Mn = fmaxf(Mn, s_red[w]);
    const float Mr = (Mn == kNegInf) ? 0.f : Mn;
    if (Mn != M && M != kNegInf) {  // earlier batches were weighed against M
      const float f = fast_exp2(M - Mr);
      den *= f;
      num.x *= f;
      num.y *= f;
      num.z *= f;
      num.w *= f;
    }
    M = Mn;
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const float w = lv[k] > 0.f ? lv[k] * fast_exp2(mv[k] - Mr) : 0.f;
      den += w;
      num.x = fmaf(w, ov[k].x, num.x);
      num.y = fmaf(w, ov[k].y, num.y);
      num.z = fmaf(w, ov[k].z, num.z);
      num.w = fmaf(w, ov[k].w, num.w);
    }
  }
  s_num[sg][c] = num;
  if (c == 0) s_den[sg] = den;
  __syncthreads();
  if (sg != 0) return;
  den = 0.f;
  num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int g = 0; g < SG; ++g) {
    const float4 o = s_num[g][c];
    num.x += o.x;
    num.y += o.y;
    num.z += o.z;
    num.w += o.w;
    den += s_den[g];
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  if constexpr (sizeof(T) == 2) {
    uint2 w;
    w.x = pack_bf16x2(num.x * inv, num.y * inv);
    w.y = pack_bf16x2(num.z * inv, num.w * inv);
    *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(a.out) + (int64_t)r * D + c * 4) = w;
  } else {
    *reinterpret_cast<float4 *>(reinterpret_cast<float *>(a.out) + (int64_t)r * D + c * 4) =
        make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv);
  }
}

// ---------------------------------------------------------------------------
// bf16, head_dim 128: the same split decode with both contractions on
// v_mfma_f32_16x16x32_bf16.  A wavefront owns (request, split, kv-head, up to
// 16 query heads of its group; unused columns are zero).  Per iteration it
// takes 32 keys:
//   S^T (keys x heads) = K Q^T   A = K rows, loaded straight from the pool in
//                                operand layout (lane c%16 <-> key, lane
//                                group <-> 8 dims), B = Q held in registers;
//   O^T (dims x heads) += V^T P^T  A = V^T, built in registers from V rows
//                                loaded whole (lane c <-> 8 dims, lane group
//                                g <-> 8 keys) by an 8 x 8 bf16 transpose,
//                                B = P^T taken from the S^T accumulators.
// Lane (c, g) = (lane % 16, lane / 16) holds S^T for keys 16t + 4g + i
// (tile t, i < 4) of head c, so a head's running max is shared across the four
// lane groups with two xor shuffles; the running sums stay per lane until the
// end.  Rows of the next iteration are in flight while the current ones are
// used.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16(const uint4 &a, const uint4 &b, const f32x4_t &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

constexpr int kMfmaD = 128;  // value width (and key width unless DK says otherwise)
constexpr int kRing = 2;     // register tile sets of a wavefront (3 and 4 measured no faster)
constexpr int kKT = 32;      // keys per iteration of a wavefront

// Online-softmax attention of one wavefront over the keys [start, end) of
// request b, for the query heads h0 .. h0 + 15 of kv-head hk (columns c with
// col_ok; the others are zero).  The workgroup stages the slot ids of up to
// kSlotTile keys at a time in LDS (all four waves take part in the barriers);
// within each staged run the wavefront takes the 32-key tiles first,
// first + TS, first + 2 TS, ...  With NEW the key at position newpos is read
// from the rows knew / vnew (this kv-head's K and V of the token written in
// the same step) instead of the pool.  pool_row is the table row the keys are
// read through (req_pool_indices of the request, read by the caller together
// with seq_lens so that the two loads share one memory round trip).  qcol is
// the query row of this lane's column (a query head of one request), or null
// for an unused column.  Runs of staged slot ids hold a.chunk keys (at most
// kSlotTile).  With STREAM the K/V rows are read with non-temporal loads.
// On return o[e][i] holds the
// unnormalised O[column c][32g + 8i + e] against the base-2 running max m_run,
// and l_tot the running sum (both per column, equal in the four lane groups).
template <int TS, bool NEW, int P, int DK = kMfmaD, bool ROPE = false, bool STREAM = false>
__device__ __forceinline__ void attend_mfma(const DecodeArgs &a, int32_t *s_slot, int pool_row,
                                            int start, int end, int first, bool active, int hk,
                                            const uint16_t *qcol, const uint16_t *knew,
                                            const uint16_t *vnew, int newpos, f32x4_t (&o)[8],
                                            float &m_run, float &l_tot,
                                            const float *rope_row = nullptr,
                                            float *s_rope = nullptr, uint16_t *rope_dst = nullptr,
                                            uint4 rope_piece = uint4{}) {
  constexpr int D = kMfmaD;  // value width
  constexpr int KS = DK / 32;  // 32-dim steps over the key width
  constexpr int KT = kKT;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int g = lane >> 4;

  // Slot ids of a staged run of keys [r0, r0 + run_cap): every thread loads
  // its SPT entries before any LDS store (one memory round trip per run).
  // The loads depend on pool_row only, not on seq_lens[b]: entries past the
  // split's end (clamped to the table row) are staged but never used.
  const int32_t *table = a.req_to_token + (int64_t)pool_row * a.table_stride;
  constexpr int SPT = kSlotTile / 256;
  const int run_cap = min(a.chunk, kSlotTile);
  int sv[SPT];
  auto load_run = [&](int r0) {
#pragma unroll
    for (int k = 0; k < SPT; ++k)
      if (256 * k < run_cap)
        sv[k] = slot_of_pos(
            table, (uint32_t)min((int64_t)r0 + (int)threadIdx.x + 256 * k, a.max_ctx_len - 1),
            a.page_shift);
  };
  auto store_run = [&]() {
#pragma unroll
    for (int k = 0; k < SPT; ++k)
      if (256 * k < run_cap) s_slot[threadIdx.x + 256 * k] = sv[k];
  };
  load_run(start);  // first on the dependent chain to the K/V rows
  // ROPE: the table row of the new token's position (DK floats), staged in
  // LDS with the first run of slot ids.
  float4 rope_v = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (ROPE) {
    static_assert(DK == kMfmaD, "rotary turn of 128-wide rows");
    static_assert(!NEW, "with the rotary turn the new rows are written, then read as pool rows");
    if (threadIdx.x < DK / 4) rope_v = reinterpret_cast<const float4 *>(rope_row)[threadIdx.x];
  }

  // Q^T operand: column c, dims 8g + 32k .. +8 for step k.
  uint4 qf[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k)
    qf[k] = (active && qcol) ? load16(qcol + 8 * g + 32 * k) : make_uint4(0u, 0u, 0u, 0u);

  const int64_t krow_elems = (int64_t)a.n_kv_heads * DK;
  const int64_t vrow_elems = (int64_t)a.n_kv_heads * D;
  const uint16_t *kbase = reinterpret_cast<const uint16_t *>(a.k_layer) + (int64_t)hk * DK + 8 * g;
  const uint16_t *vbase = reinterpret_cast<const uint16_t *>(a.v_layer) + (int64_t)hk * D + 8 * c;
  const uint16_t *knew_l = NEW ? knew + 8 * g : nullptr;
  const uint16_t *vnew_l = NEW ? vnew + 8 * c : nullptr;

#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  m_run = kNegInf;     // base-2 running max of head c (same in all four groups)
  float l_lane = 0.f;  // this lane's share of the running sum

  // K rows: keys 16t + c (t < 2), 16 bytes at dims 8g + 32k.  V rows: keys
  // 4g + i and 16 + 4g + i (i < 4), dims 8c .. 8c + 7.  Tokens past the end
  // of the round read the round's last row instead (finite data whose score is
  // masked to -inf, so its weight is 0): the loads stay unconditional, which
  // lets the compiler keep several tiles in flight.
  auto row16 = [](const uint16_t *p) {
    if constexpr (STREAM)
      return load16_nt(p);
    else
      return load16(p);
  };
  auto fetch = [&](uint4(&kx)[2][KS], uint4(&vx)[8], int j0, int r0, int r1) {
    const int last = r1 - 1 - r0;
    const int jb = j0 - r0;
    int jk[2], jv[8];
#pragma unroll
    for (int t = 0; t < 2; ++t) jk[t] = min(jb + 16 * t + c, last);
#pragma unroll
    for (int x = 0; x < 8; ++x) jv[x] = min(jb + 16 * (x >> 2) + 4 * g + (x & 3), last);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint16_t *kp = kbase + (int64_t)s_slot[jk[t]] * krow_elems;
      if constexpr (NEW) kp = (r0 + jk[t] == newpos) ? knew_l : kp;
#pragma unroll
      for (int k = 0; k < KS; ++k) kx[t][k] = row16(kp + 32 * k);
    }
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const uint16_t *vp = vbase + (int64_t)s_slot[jv[x]] * vrow_elems;
      if constexpr (NEW) vp = (r0 + jv[x] == newpos) ? vnew_l : vp;
      vx[x] = row16(vp);
    }
  };

  auto process = [&](const uint4(&kx)[2][KS], const uint4(&vx)[8], int j0, int r1) {
    f32x4_t st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      st[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KS; ++k) st[t] = mfma16(kx[t][k], qf[k], st[t]);
    }
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = j0 + 16 * t + 4 * g + i < r1;
        st[t][i] = ok ? st[t][i] * a.scale_log2 : kNegInf;
        mx = fmaxf(mx, st[t][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float mref = (m_new == kNegInf) ? 0.f : m_new;
    if (__any(m_new != m_run)) {  // rescale only when some head's max moved
      const float alpha = fast_exp2(m_run - mref);
      l_lane *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] *= alpha;
    }
    m_run = m_new;
    float p[8];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[4 * t + i] = fast_exp2(st[t][i] - mref);
        l_lane += p[4 * t + i];
      }
    uint4 pf;
    pf.x = pack_bf16x2(p[0], p[1]);
    pf.y = pack_bf16x2(p[2], p[3]);
    pf.z = pack_bf16x2(p[4], p[5]);
    pf.w = pack_bf16x2(p[6], p[7]);
    // V^T operand e: element x is dim 8c + e of key x's row.
    const uint32_t w[8][4] = {
        {vx[0].x, vx[0].y, vx[0].z, vx[0].w}, {vx[1].x, vx[1].y, vx[1].z, vx[1].w},
        {vx[2].x, vx[2].y, vx[2].z, vx[2].w}, {vx[3].x, vx[3].y, vx[3].z, vx[3].w},
        {vx[4].x, vx[4].y, vx[4].z, vx[4].w}, {vx[5].x, vx[5].y, vx[5].z, vx[5].w},
        {vx[6].x, vx[6].y, vx[6].z, vx[6].w}, {vx[7].x, vx[7].y, vx[7].z, vx[7].w}};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t d[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint32_t lo = w[2 * x][e >> 1], hi = w[2 * x + 1][e >> 1];
        d[x] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      o[e] = mfma16(make_uint4(d[0], d[1], d[2], d[3]), pf, o[e]);
    }
  };

  // Ring of P register tile sets: P - 1 tiles are in flight while one is used.
  static_assert(P >= 2, "pipeline depth");
  uint4 kr[P][2][KS], vr[P][8];
  // Rounds of run_cap keys: a split of up to one chunk takes one round (or
  // rounds of kSlotTile), the last split's tail past num_splits * chunk more.
  for (int r0 = start; r0 < end; r0 += run_cap) {
    const int r1 = min(end, r0 + run_cap);
    if (r0 != start) {
      __syncthreads();
      load_run(r0);
    }
    store_run();
    if constexpr (ROPE) {
      if (r0 == start && threadIdx.x < DK / 4)
        reinterpret_cast<float4 *>(s_rope)[threadIdx.x] = rope_v;
    }
    __syncthreads();
    if constexpr (ROPE) {
      if (r0 == start) {
#pragma unroll
        for (int k = 0; k < KS; ++k) qf[k] = rotate_bf16x8(qf[k], s_rope + 8 * g + 32 * k);
        // The new token's rows, written before any of them is fetched: lanes
        // [0, DK/8) carry the key pieces (turned here), the next D/8 lanes the
        // value pieces.  This wave is the only reader of its kv-head's rows of
        // the split; the release / acquire pair orders the other lanes' later
        // loads of those rows after the stores.
        if (rope_dst) {
          const uint4 piece =
              lane < DK / 8 ? rotate_bf16x8(rope_piece, s_rope + 8 * lane) : rope_piece;
          store16(rope_dst, piece);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      }
    }
    if (!active) continue;
    const int round_tiles = (r1 - r0 + KT - 1) / KT;
    const int ntiles = first < round_tiles ? (round_tiles - first + TS - 1) / TS : 0;
    auto j0_of = [&](int i) { return r0 + (first + i * TS) * KT; };
#pragma unroll
    for (int q = 0; q < P - 1; ++q) fetch(kr[q], vr[q], j0_of(q), r0, r1);
    int i = 0;
    for (; i + P <= ntiles; i += P) {
#pragma unroll
      for (int q = 0; q < P; ++q) {
        fetch(kr[(q + P - 1) % P], vr[(q + P - 1) % P], j0_of(i + q + P - 1), r0, r1);
        process(kr[q], vr[q], j0_of(i + q), r1);
      }
    }
#pragma unroll
    for (int q = 0; q < P - 1; ++q)
      if (i + q < ntiles) process(kr[q], vr[q], j0_of(i + q), r1);
  }
  l_tot = l_lane + __shfl_xor(l_lane, 16);
  l_tot += __shfl_xor(l_tot, 32);
}

// With NEW the launch also completes the step's K/V write: the new token's
// rows (position seq_lens[b] - 1) are attended straight from k_new / v_new,
// and the wavefront of head chunk 0 of each kv-head in the split holding that
// position writes them to the pool slot out_cache_loc[b] (no wavefront of
// the launch reads that pool row).
// With ROPE (NEW only) q and k_new arrive unrotated: every wavefront turns
// its query rows by row position_ids[b] of the table (staged in s_rope), and
// the wavefront of each kv-head in the split holding the new token writes the
// turned key row and the value row to the pool before it fetches any row, so
// the split reads them as pool rows (one wavefront per kv-head: at most 16
// query heads per kv-head, and out_cache_loc[b] the slot of position
// seq_lens[b] - 1).
template <bool NEW, int DK = kMfmaD, bool ROPE = false, bool STREAM = false>
__device__ __forceinline__ void split_mfma_body(const StepArgs &sa, int32_t *s_slot, int b, int s,
                                                int wx, float *s_rope = nullptr) {
  constexpr int D = kMfmaD;  // value width; keys are DK wide
  const DecodeArgs &a = sa.d;
  static_assert(!ROPE || NEW, "the rotary turn comes with the new-token write");

  const int L = a.seq_lens[b];
  const int pool_row = a.req_pool_indices[b];
  const float *rope_row = nullptr;
  if constexpr (ROPE) {
    const int64_t p = min(max((int64_t)sa.position_ids[b], (int64_t)0), sa.max_pos - 1);
    rope_row = sa.freqs + p * D;
  }
  // With a shared prefix the request's own splits start at kv_start[b].
  const int start = (a.kv_start ? a.kv_start[b] : 0) + s * a.chunk;
  const int end = split_end(a, s, start, L);

  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int task = wx * 4 + (threadIdx.x >> 6);
  const bool active = task < a.n_kv_heads * a.n_chunks;
  const int hk = active ? task / a.n_chunks : 0;
  const int g0 = active ? (task - hk * a.n_chunks) * a.heads_per_chunk : 0;
  const int ng = active ? min(a.heads_per_chunk, a.group - g0) : 0;
  const int h0 = hk * a.group + g0;
  const bool col_ok = c < ng;
  const int S = a.split_stride;
  const int64_t pr = ((int64_t)b * a.n_heads + h0 + c) * S + s;  // partial row of head h0 + c

  const int newpos = NEW ? L - 1 : -1;
  const uint16_t *knew = nullptr, *vnew = nullptr;
  // The new token's rows for the pool write: loaded here, stored after the
  // attention, so the write adds no wait to this split's start-up chain.
  bool writer = false;
  uint4 new_piece = make_uint4(0u, 0u, 0u, 0u);
  uint16_t *new_dst = nullptr;
  if constexpr (NEW) {
    const int64_t row = (int64_t)b * a.n_kv_heads + hk;  // row of k_new / v_new
    knew = reinterpret_cast<const uint16_t *>(sa.k_new) + row * DK;
    vnew = reinterpret_cast<const uint16_t *>(sa.v_new) + row * D;
    // lanes [0, DK/8) carry the key row's 16-byte pieces, the next D/8 lanes
    // the value row's
    writer = active && g0 == 0 && start <= newpos && newpos < end && lane < (DK + D) / 8;
    if (writer) {
      const int64_t loc = sa.out_cache_loc[b];
      const bool is_k = lane < DK / 8;
      const int piece = is_k ? lane : lane - DK / 8;
      new_piece = load16((is_k ? knew : vnew) + 8 * piece);
      new_dst = is_k ? reinterpret_cast<uint16_t *>(sa.k_layer_w) +
                           (loc * a.n_kv_heads + hk) * DK + 8 * piece
                     : reinterpret_cast<uint16_t *>(sa.v_layer_w) +
                           (loc * a.n_kv_heads + hk) * D + 8 * piece;
    }
  }

  // An empty split (start >= end, splits past a short request's length)
  // writes the empty state o = 0, m = -inf, l = 0 and leaves before staging
  // any slot id.  The asm operands make the length and the table row address
  // ready before the branch, so the seq_lens[b], req_pool_indices[b] and
  // table-argument loads all issue before it (an exit that needs only
  // seq_lens[b] would let the compiler issue the others after it, lengthening
  // the start-up chain of every non-empty split).
  const int32_t *table_row = a.req_to_token + (int64_t)pool_row * a.table_stride;
  asm volatile("" ::"s"(L), "s"(table_row), "s"(a.page_shift), "s"(a.max_ctx_len), "s"(start));
  if (start >= end) {
    const bool bad = split_overrun(a, L);
    // With skip_empty the merge reads only the splits that hold keys.
    if (a.skip_empty && !bad) return;
    const float ov = bad ? NAN : 0.f;
    if (active && col_ok) {
      float4 *op = reinterpret_cast<float4 *>(a.o_part + pr * D + 32 * g);
#pragma unroll
      for (int i = 0; i < 8; ++i) op[i] = make_float4(ov, ov, ov, ov);
      if (g == 0) {
        a.ml_part[pr * 2 + 0] = bad ? NAN : kNegInf;
        a.ml_part[pr * 2 + 1] = bad ? 1.f : 0.f;
      }
    }
    return;
  }
  f32x4_t o[8];
  float m_run, l_tot;
  // Only the split holding the new token substitutes its rows in the fetch;
  // every other split runs the plain loop.
  const uint16_t *qcol =
      col_ok ? reinterpret_cast<const uint16_t *>(a.q) + ((int64_t)b * a.n_heads + h0 + c) * DK
             : nullptr;
  if constexpr (ROPE) {
    // The new rows go to the pool first (turned key, value), then every
    // split reads pool rows only.
    attend_mfma<1, false, kRing, DK, true, STREAM>(a, s_slot, pool_row, start, end, 0, active, hk, qcol,
                                           nullptr, nullptr, -1, o, m_run, l_tot, rope_row,
                                           s_rope, writer ? new_dst : nullptr, new_piece);
  } else if (NEW && start <= newpos && newpos < end) {
    attend_mfma<1, true, kRing, DK, false, STREAM>(a, s_slot, pool_row, start, end, 0, active, hk,
                                                   qcol, knew,
                                    vnew, newpos, o, m_run, l_tot);
  } else {
    attend_mfma<1, false, kRing, DK, false, STREAM>(a, s_slot, pool_row, start, end, 0, active,
                                                    hk, qcol, nullptr, nullptr, -1, o, m_run,
                                                    l_tot);
  }
  if (NEW && !ROPE && writer) store16(new_dst, new_piece);
  if (!active || !col_ok) return;
  // Lane (c, g) holds O[head c][32g + 8i + e] in o[e][i].
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  float4 *op = reinterpret_cast<float4 *>(a.o_part + pr * D + 32 * g);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    op[2 * i + 0] = make_float4(o[0][i] * inv, o[1][i] * inv, o[2][i] * inv, o[3][i] * inv);
    op[2 * i + 1] = make_float4(o[4][i] * inv, o[5][i] * inv, o[6][i] * inv, o[7][i] * inv);
  }
  if (g == 0) {
    a.ml_part[pr * 2 + 0] = m_run;
    a.ml_part[pr * 2 + 1] = l_tot;
  }
}

// Keys 192 wide (MLA-shaped layers) hold more registers per wavefront: one
// wavefront per SIMD, instead of two for 128-wide keys.
template <bool NEW, int DK, bool STREAM>
__global__ void __launch_bounds__(256, DK == 128 ? 2 : 1) decode_split_mfma_kernel(const StepArgs sa) {
  __shared__ int32_t s_slot[kSlotTile];
  split_mfma_body<NEW, DK, false, STREAM>(sa, s_slot, blockIdx.z, blockIdx.y, blockIdx.x);
}

// The split kernel with the new-token write and the rotary turn of q and
// k_new (bf16, keys and values 128 wide).
template <bool STREAM>
__global__ void __launch_bounds__(256, 2) decode_split_rope_kernel(const StepArgs sa) {
  __shared__ int32_t s_slot[kSlotTile];
  __shared__ __align__(16) float s_rope[kMfmaD];  // the table row of the new token
  split_mfma_body<true, kMfmaD, true, STREAM>(sa, s_slot, blockIdx.z, blockIdx.y, blockIdx.x,
                                              s_rope);
}

// ---------------------------------------------------------------------------
// Shared-prefix decode (bf16, head_dim 128).  The members of a prefix group
// read the same slots for their first P positions, so those keys are
// gathered once per group: a wavefront owns (group, prefix split, kv-head,
// 16 columns), where the columns enumerate (member, query head of the
// kv-head's group) as member * G + head, and it runs the same matrix-core
// routine as the split kernel with those columns as the query rows.  Each
// column's (m, l, o) partial goes to its member's partial row, after the
// member's own num_splits splits (which the split kernel runs over keys
// [kv_start[b], seq_lens[b]) = [P, seq_lens[b])).  The merge weighs both.
__device__ __forceinline__ void prefix_mfma_body(const PrefixArgs &pa, int32_t *s_slot, int grp,
                                                 int s, int wx) {
  constexpr int D = kMfmaD;
  const DecodeArgs &a = pa.d;

  const int32_t *rec = pa.groups + (int64_t)grp * pa.group_ints;
  const int P = rec[0];
  const int m = rec[1];
  const int pool_row = a.req_pool_indices[rec[2]];  // any member's row: same slots below P
  const int start = s * a.chunk;
  const int end = s == pa.prefix_splits - 1 ? P : min(P, start + a.chunk);

  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int G = a.group;
  const int n_cc = (m * G + 15) >> 4;  // 16-column chunks of this group per kv-head
  const int task = wx * 4 + (threadIdx.x >> 6);
  const bool active = task < a.n_kv_heads * n_cc;
  const int hk = active ? task / n_cc : 0;
  const int idx = (active ? task - hk * n_cc : 0) * 16 + c;
  const int member = idx / G;
  const bool col_ok = active && member < m;
  const int bm = col_ok ? rec[2 + member] : 0;
  const int head = hk * G + (idx - member * G);
  const int64_t pr = ((int64_t)bm * a.n_heads + head) * a.split_stride + a.num_splits + s;

  const int32_t *table_row = a.req_to_token + (int64_t)pool_row * a.table_stride;
  asm volatile("" ::"s"(P), "s"(table_row), "s"(a.page_shift), "s"(a.max_ctx_len));
  if (start >= end) {  // a split past this group's prefix: the empty partial
    if (a.skip_empty) return;
    if (col_ok) {
      float4 *op = reinterpret_cast<float4 *>(a.o_part + pr * D + 32 * g);
#pragma unroll
      for (int i = 0; i < 8; ++i) op[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (g == 0) {
        a.ml_part[pr * 2 + 0] = kNegInf;
        a.ml_part[pr * 2 + 1] = 0.f;
      }
    }
    return;
  }
  const uint16_t *qcol =
      col_ok ? reinterpret_cast<const uint16_t *>(a.q) + ((int64_t)bm * a.n_heads + head) * D
             : nullptr;
  f32x4_t o[8];
  float m_run, l_tot;
  attend_mfma<1, false, kRing>(a, s_slot, pool_row, start, end, 0, active, hk, qcol, nullptr,
                               nullptr, -1, o, m_run, l_tot);
  if (!col_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  float4 *op = reinterpret_cast<float4 *>(a.o_part + pr * D + 32 * g);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    op[2 * i + 0] = make_float4(o[0][i] * inv, o[1][i] * inv, o[2][i] * inv, o[3][i] * inv);
    op[2 * i + 1] = make_float4(o[4][i] * inv, o[5][i] * inv, o[6][i] * inv, o[7][i] * inv);
  }
  if (g == 0) {
    a.ml_part[pr * 2 + 0] = m_run;
    a.ml_part[pr * 2 + 1] = l_tot;
  }
}

__global__ void __launch_bounds__(256, 2) decode_prefix_mfma_kernel(const PrefixArgs pa) {
  __shared__ int32_t s_slot[kSlotTile];
  prefix_mfma_body(pa, s_slot, blockIdx.z, blockIdx.y, blockIdx.x);
}

// The whole shared-prefix attention in one launch: the groups' shared keys
// (workgroups 0 .. pfx_blocks - 1, dispatched first: each takes a longer
// run of keys) and every request's own keys with the new token's K/V write.
__global__ void __launch_bounds__(256, 2) decode_shared_mfma_kernel(const SharedArgs sh) {
  __shared__ int32_t s_slot[kSlotTile];
  int lin = blockIdx.x;
  if (lin < sh.pfx_blocks) {
    const int wx = lin % sh.pfx_wx;
    const int rest = lin / sh.pfx_wx;
    const int s = rest % sh.pfx.prefix_splits;
    prefix_mfma_body(sh.pfx, s_slot, rest / sh.pfx.prefix_splits, s, wx);
  } else {
    lin -= sh.pfx_blocks;
    const int wx = lin % sh.sfx_wx;
    const int rest = lin / sh.sfx_wx;
    const int s = rest % sh.sfx.d.num_splits;
    split_mfma_body<true>(sh.sfx, s_slot, rest / sh.sfx.d.num_splits, s, wx);
  }
}

// ---------------------------------------------------------------------------
// One decode step in one launch (bf16, head_dim 128): the K/V write of every
// request's new token, the split attention and the merge (the three steps of
// the "KVCache System" write plus the "Attention Backend" decode call).
// A workgroup owns (request b, task = kv-head and chunk of <= 16 of its query
// heads, split s); its four waves take interleaved 32-key tiles of the split
// and combine their (m, l, o) states in LDS into one split partial, written
// in the workspace format of the split kernel.  The new token's K/V rows are
// read from k_new / v_new (the workgroup of the split holding the token also
// writes them to the pool; nothing in this launch reads that pool row).  Each
// workgroup then takes a ticket on the (b, task) counter in sync; the last of
// the num_splits workgroups merges the task's partials into out and resets
// the counter to zero.
// Relaxed device-scope (agent) accesses: coherent across the XCDs' L2s
// without the whole-cache write-back and invalidate of a device fence.
__device__ __forceinline__ void store_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(15): wait for this wave's vector
// memory operations only.
constexpr int kWaitVmem0 = 0x0F70;
__global__ void __launch_bounds__(256, 2) decode_step_kernel(const StepArgs sa) {
  constexpr int D = kMfmaD;
  const DecodeArgs &a = sa.d;
  // LDS: slot ids while attending, then the four waves' states.
  __shared__ __align__(16) char s_raw[4 * 16 * D * 4 + 2 * 4 * 16 * 4];
  __shared__ int s_last;
  int32_t *s_slot = reinterpret_cast<int32_t *>(s_raw);
  static_assert(kSlotTile * 4 <= 4 * 16 * D * 4, "LDS reuse");
  float *s_o = reinterpret_cast<float *>(s_raw);       // [wave][head][dim]
  float *s_m = s_o + 4 * 16 * D;                       // [wave][head]
  float *s_l = s_m + 4 * 16;                           // [wave][head]

  const int b = blockIdx.z;
  const int s = blockIdx.y;
  const int task = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int L = a.seq_lens[b];
  const int pool_row = a.req_pool_indices[b];
  const int start = s * a.chunk;
  const int end = split_end(a, s, start, L);
  const int hk = task / a.n_chunks;
  const int chunk_i = task - hk * a.n_chunks;
  const int g0 = chunk_i * a.heads_per_chunk;
  const int ng = min(a.heads_per_chunk, a.group - g0);
  const int h0 = hk * a.group + g0;
  const int S = a.num_splits;
  const int newpos = L - 1;
  const int64_t new_row = ((int64_t)b * a.n_kv_heads + hk) * D;  // element offset in k_new / v_new
  const uint16_t *knew = reinterpret_cast<const uint16_t *>(sa.k_new) + new_row;
  const uint16_t *vnew = reinterpret_cast<const uint16_t *>(sa.v_new) + new_row;

  // The pool write of the new token's row of this kv-head (once per kv-head).
  if (chunk_i == 0 && start <= newpos && newpos < end && tid < 2 * D / 8) {
    const int64_t loc = sa.out_cache_loc[b];
    const int64_t dst = (loc * a.n_kv_heads + hk) * D + 8 * (tid & 15);
    if (tid < D / 8)
      store16(reinterpret_cast<uint16_t *>(sa.k_layer_w) + dst, load16(knew + 8 * (tid & 15)));
    else
      store16(reinterpret_cast<uint16_t *>(sa.v_layer_w) + dst, load16(vnew + 8 * (tid & 15)));
  }

  f32x4_t o[8];
  float m_run, l_tot;
  const uint16_t *qcol =
      c < ng ? reinterpret_cast<const uint16_t *>(a.q) + ((int64_t)b * a.n_heads + h0 + c) * D
             : nullptr;
  attend_mfma<4, true, kRing>(a, s_slot, pool_row, start, end, wave, true, hk, qcol, knew, vnew,
                              newpos, o, m_run, l_tot);

  // Combine the four waves' states into the split partial.
  __syncthreads();  // slot ids are dead
  if (c < ng) {
    float *wo = s_o + (wave * 16 + c) * D + 32 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<float4 *>(wo + 8 * i) = make_float4(o[0][i], o[1][i], o[2][i], o[3][i]);
      *reinterpret_cast<float4 *>(wo + 8 * i + 4) = make_float4(o[4][i], o[5][i], o[6][i], o[7][i]);
    }
    if (g == 0) {
      s_m[wave * 16 + c] = m_run;
      s_l[wave * 16 + c] = l_tot;
    }
  }
  __syncthreads();
  {
    const int hc = tid >> 4;        // head column
    const int d0 = (tid & 15) * 8;  // 8 dims
    if (hc < ng) {
      float mw[4], lw[4];
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        mw[w] = s_m[w * 16 + hc];
        lw[w] = s_l[w * 16 + hc];
        if (lw[w] > 0.f) M = fmaxf(M, mw[w]);
      }
      float f[4], lsum = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        f[w] = lw[w] > 0.f ? fast_exp2(mw[w] - M) : 0.f;
        lsum = fmaf(f[w], lw[w], lsum);
      }
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (f[w] == 0.f) continue;  // an empty wave's o is never read
        const float *wo = s_o + (w * 16 + hc) * D + d0;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(f[w], wo[e], acc[e]);
      }
      // Device-scope stores: the partial is read by whichever workgroup (on
      // any XCD) merges, so it must not wait in this XCD's L2.
      // A request past max_ctx_len attended nothing: its partial is NaN.
      const bool bad = split_overrun(a, L);
      const int64_t pr = ((int64_t)b * a.n_heads + h0 + hc) * S + s;
      float *op = a.o_part + pr * D + d0;
#pragma unroll
      for (int e = 0; e < 8; ++e) store_agent(op + e, bad ? NAN : acc[e] * inv);
      if ((tid & 15) == 0) {
        store_agent(a.ml_part + pr * 2 + 0, bad ? NAN : (lsum > 0.f ? M : kNegInf));
        store_agent(a.ml_part + pr * 2 + 1, bad ? 1.f : lsum);
      }
    }
  }

  // Ticket: the last split of (b, task) to finish merges.  The hand-off is
  // a release / acquire pair at agent scope: the workgroup barrier orders
  // every thread's partial stores before thread 0's ticket, the ticket is an
  // agent-scope release read-modify-write, and the workgroup that draws the
  // last ticket issues an agent-scope acquire fence before it reads any
  // partial.  By the HIP memory model the merging workgroup therefore sees
  // every partial of the (b, task) row, whichever XCD wrote it.  Each wave
  // also waits for its own partial stores to complete before the barrier
  // (s_waitcnt vmcnt(0)), so the ticket is never drawn while a store of the
  // workgroup is still in flight.
  __builtin_amdgcn_s_waitcnt(kWaitVmem0);
  __syncthreads();
  if (tid == 0) {
    const int t = __hip_atomic_fetch_add(&sa.sync[(int64_t)b * sa.tasks + task], 1,
                                         __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    s_last = t == S - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  // Merge: wave w takes heads w, w + 4, ...; lane l dims 2l, 2l + 1.  Up to
  // 32 splits per memory round trip.
  constexpr int KB = 32;
  for (int hc = wave; hc < ng; hc += 4) {
    const int64_t row = (int64_t)b * a.n_heads + h0 + hc;
    const float *ml = a.ml_part + row * S * 2;
    const float *op = a.o_part + row * S * D + 2 * lane;
    float M = kNegInf, den = 0.f, n0 = 0.f, n1 = 0.f;
    for (int s0 = 0; s0 < S; s0 += KB) {
      float mv[KB], lv[KB];
      float2 ov[KB];
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int sk = min(s0 + k, S - 1);
        mv[k] = load_agent(ml + 2 * sk);
        lv[k] = s0 + k < S ? load_agent(ml + 2 * sk + 1) : 0.f;
        ov[k] = make_float2(load_agent(op + (int64_t)sk * D), load_agent(op + (int64_t)sk * D + 1));
      }
      float bm = M;
#pragma unroll
      for (int k = 0; k < KB; ++k)
        if (lv[k] > 0.f) bm = fmaxf(bm, mv[k]);
      if (bm != M && M != kNegInf) {  // earlier batches were weighed against M
        const float f = fast_exp2(M - bm);
        den *= f;
        n0 *= f;
        n1 *= f;
      }
      M = bm;
      const float Mr = (M == kNegInf) ? 0.f : M;
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const float w = lv[k] > 0.f ? lv[k] * fast_exp2(mv[k] - Mr) : 0.f;
        den += w;
        n0 = fmaf(w, ov[k].x, n0);
        n1 = fmaf(w, ov[k].y, n1);
      }
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    *reinterpret_cast<uint32_t *>(reinterpret_cast<uint16_t *>(sa.out) + row * D + 2 * lane) =
        pack_bf16x2(n0 * inv, n1 * inv);
  }
  if (tid == 0)
    __hip_atomic_store(&sa.sync[(int64_t)b * sa.tasks + task], 0, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
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

// Few rows (a decode step of few requests): 256 threads with batches of 16
// splits per thread, one memory round trip for up to 128 splits of 128-dim
// rows.  Many rows: 128 threads with batches of 12 (48 splits of 128-dim
// rows per round trip), small enough that every row of a 2048-row step is
// resident at once (a 256-thread workgroup per row left a third of them for
// a second round).
template <typename T, int D>
void merge_d(const MergeArgs &a, hipStream_t stream) {
  if (a.rows > 1024)
    hipLaunchKernelGGL((decode_merge_kernel<T, D, 12, 128>), dim3(a.rows), dim3(128), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_merge_kernel<T, D, 16, 256>), dim3(a.rows), dim3(256), 0, stream, a);
}

}  // namespace

bool decode_mfma_shape(int dtype, int head_dim, int v_head_dim) {
  return dtype == 1 && v_head_dim == kMfmaD && (head_dim == 128 || head_dim == 192);
}

// The matrix-core split kernel for the key width and load kind of sa.
template <bool NEW>
void split_d(const StepArgs &sa, int head_dim, dim3 grid, hipStream_t stream) {
  const bool st = sa.d.stream_rows != 0;
  if (head_dim == 192 && st)
    hipLaunchKernelGGL((decode_split_mfma_kernel<NEW, 192, true>), grid, dim3(256), 0, stream, sa);
  else if (head_dim == 192)
    hipLaunchKernelGGL((decode_split_mfma_kernel<NEW, 192, false>), grid, dim3(256), 0, stream, sa);
  else if (st)
    hipLaunchKernelGGL((decode_split_mfma_kernel<NEW, 128, true>), grid, dim3(256), 0, stream, sa);
  else
    hipLaunchKernelGGL((decode_split_mfma_kernel<NEW, 128, false>), grid, dim3(256), 0, stream, sa);
}

hipError_t launch_paged_decode(const DecodeArgs &args, int dtype, int head_dim, int v_head_dim,
                               hipStream_t stream) {
  DecodeArgs a = args;
  // Query heads of a kv-head's group served by one wavefront: up to 16 on the
  // matrix-core path (bf16, values 128 wide, keys 128 or 192), up to 8 on the
  // vector path.
  const bool mfma = decode_mfma_shape(dtype, head_dim, v_head_dim);
  const int per_wave = mfma ? 16 : 8;
  a.n_chunks = (a.group + per_wave - 1) / per_wave;
  a.heads_per_chunk = (a.group + a.n_chunks - 1) / a.n_chunks;
  if (mfma) {
    StepArgs sa{};
    sa.d = a;
    const dim3 grid((a.n_kv_heads * a.n_chunks + 3) / 4, a.num_splits, a.batch);
    split_d<false>(sa, head_dim, grid, stream);
    return hipGetLastError();
  }
  if (head_dim != v_head_dim) return hipErrorInvalidValue;
  if (dtype == 1) {
    if (head_dim == 128) return decode_dispatch_ng<uint16_t, 128>(a, stream);
    if (head_dim == 64) return decode_dispatch_ng<uint16_t, 64>(a, stream);
  } else {
    if (head_dim == 128) return decode_dispatch_ng<float, 128>(a, stream);
    if (head_dim == 64) return decode_dispatch_ng<float, 64>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_step(const StepArgs &args, hipStream_t stream) {
  StepArgs sa = args;
  DecodeArgs &a = sa.d;
  a.n_chunks = (a.group + 15) / 16;
  a.heads_per_chunk = (a.group + a.n_chunks - 1) / a.n_chunks;
  sa.tasks = a.n_kv_heads * a.n_chunks;
  const dim3 grid(sa.tasks, a.num_splits, a.batch);
  hipLaunchKernelGGL(decode_step_kernel, grid, dim3(256), 0, stream, sa);
  return hipGetLastError();
}

hipError_t launch_decode_split_store(const StepArgs &args, int head_dim, hipStream_t stream) {
  StepArgs sa = args;
  DecodeArgs &a = sa.d;
  a.n_chunks = (a.group + 15) / 16;
  a.heads_per_chunk = (a.group + a.n_chunks - 1) / a.n_chunks;
  const dim3 grid((a.n_kv_heads * a.n_chunks + 3) / 4, a.num_splits, a.batch);
  split_d<true>(sa, head_dim, grid, stream);
  return hipGetLastError();
}

hipError_t launch_decode_split_rope(const StepArgs &args, hipStream_t stream) {
  StepArgs sa = args;
  DecodeArgs &a = sa.d;
  a.n_chunks = (a.group + 15) / 16;
  a.heads_per_chunk = (a.group + a.n_chunks - 1) / a.n_chunks;
  const dim3 grid((a.n_kv_heads * a.n_chunks + 3) / 4, a.num_splits, a.batch);
  if (a.stream_rows)
    hipLaunchKernelGGL(decode_split_rope_kernel<true>, grid, dim3(256), 0, stream, sa);
  else
    hipLaunchKernelGGL(decode_split_rope_kernel<false>, grid, dim3(256), 0, stream, sa);
  return hipGetLastError();
}

hipError_t launch_decode_shared(const SharedArgs &args, hipStream_t stream) {
  SharedArgs sh = args;
  DecodeArgs &a = sh.sfx.d;
  a.n_chunks = (a.group + 15) / 16;
  a.heads_per_chunk = (a.group + a.n_chunks - 1) / a.n_chunks;
  sh.sfx_wx = (a.n_kv_heads * a.n_chunks + 3) / 4;
  const int n_cc = (sh.pfx.max_members * sh.pfx.d.group + 15) / 16;
  sh.pfx_wx = (sh.pfx.d.n_kv_heads * n_cc + 3) / 4;
  const int64_t pfx_blocks = (int64_t)sh.pfx_wx * sh.pfx.prefix_splits * sh.pfx.n_groups;
  const int64_t blocks = pfx_blocks + (int64_t)sh.sfx_wx * a.num_splits * a.batch;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  sh.pfx_blocks = (int32_t)pfx_blocks;
  hipLaunchKernelGGL(decode_shared_mfma_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, sh);
  return hipGetLastError();
}

hipError_t launch_decode_prefix(const PrefixArgs &args, hipStream_t stream) {
  PrefixArgs pa = args;
  const int n_cc = (args.max_members * args.d.group + 15) / 16;
  const dim3 grid((args.d.n_kv_heads * n_cc + 3) / 4, args.prefix_splits, args.n_groups);
  hipLaunchKernelGGL(decode_prefix_mfma_kernel, grid, dim3(256), 0, stream, pa);
  return hipGetLastError();
}

hipError_t launch_decode_merge(const MergeArgs &a, int dtype, int head_dim, hipStream_t stream) {
  if (dtype == 1) {
    if (head_dim == 128)
      merge_d<uint16_t, 128>(a, stream);
    else
      merge_d<uint16_t, 64>(a, stream);
  } else {
    if (head_dim == 128)
      merge_d<float, 128>(a, stream);
    else
      merge_d<float, 64>(a, stream);
  }
  return hipGetLastError();
}

}  // namespace pkv

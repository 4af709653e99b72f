// Ragged causal paged prefill on bf16 matrix cores (gfx950).
//
// What is computed (AstrAI "Inference" guide, section "Attention Backend"):
// after this forward's K/V are written, request i's q_len_i new tokens attend
// over its kv_len_i keys, read straight from the flat pool through
// req_to_token; q_len_i and kv_len_i come from qo_indptr and kv_indptr.  The
// t-th new token sits at logical position p_i + t, p_i = kv_len_i - q_len_i,
// and with the causal mask it sees keys 0 .. p_i + t.  Each output row is
// o = sum_j softmax_j(q . k_j * sm_scale) v_j (section "KV Cache").
//
// Tiling.  A workgroup (4 wavefronts) owns one (request, kv-head, block of 128
// query rows), where the rows of a request enumerate (token t, head g of the
// kv-head's group) as r = t * G + g, so all G query heads sharing a kv-head
// reuse one K/V tile and any group size works.  Each wavefront owns 32 rows.
// Keys stream through LDS in tiles of 64, gathered by slot:
//   S^T (keys x rows) = K Q^T : v_mfma_f32_32x32x16_bf16, A = K rows from LDS,
//                               B = the wave's Q rows held in registers;
//   O^T (dims x rows) += V^T P^T : A = V^T from LDS (V is stored transposed),
//                               B = the softmax weights, rounded to bf16,
//                               taken straight from the S^T accumulators.
// With S^T in this orientation every lane holds one query row, so the
// online-softmax row max / row sum need one cross-lane step (lane l ^ 32).
// The next tile's K/V rows are fetched into registers while the current tile
// is being multiplied.
#include <math.h>

#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace pkv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kNegInf = -INFINITY;
constexpr int NT = 256;   // threads per workgroup (4 wavefronts)
constexpr int BM = NT / 64 * 32;  // query rows per workgroup
constexpr int BN = 64;    // keys per tile
constexpr int WROWS = 32; // query rows per wavefront

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4 &v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ f32x16_t mfma32(const uint4 &a, const uint4 &b, const f32x16_t &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Position of key k of a 64-key tile inside a transposed V row: bits 2 and 3 of
// the key index are swapped, so that the eight keys one lane feeds to a PV
// product (keys 16t + {0..3, 8..11} or 16t + {4..7, 12..15}) are contiguous.
__device__ __forceinline__ int vpos(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <int D>
struct Smem {
  static constexpr int KS = D + 8;   // K row stride (elements), 16-byte pad
  static constexpr int VS = BN + 8;  // V^T row stride (elements), 16-byte pad
  uint16_t k[BN * KS];
  uint16_t vt[D * VS];
};

// OFF32: every row of the layer lies within 4 GiB of the layer base, so row
// addresses are a uniform 64-bit base plus a 32-bit byte offset.
template <int D, bool OFF32>
__global__ void __launch_bounds__(NT, 2) prefill_kernel(const PrefillArgs a) {
  constexpr int KS = Smem<D>::KS;
  constexpr int VS = Smem<D>::VS;
  constexpr int KSTEPS = D / 16;             // MFMA steps over head_dim for S^T
  constexpr int DBLK = D / 32;               // 32-dim blocks of O^T
  constexpr int KPIECES = BN * D / 8 / NT;   // 16-byte K pieces per thread per tile
  constexpr int VJOBS = (BN / 4) * (D / 8);  // (4-key, 8-dim) V jobs per tile
  __shared__ Smem<D> sm[2];  // tile n is used from one while tile n+1 is staged into the other

  // Workgroups are dispatched to the 8 XCDs round-robin by linear id; taking
  // the kv-head from the low part of the id keeps every workgroup of one
  // kv-head on the same XCD (for 8 kv-heads), so the row blocks of a request
  // share that head's K/V rows in one L2.
  const int lin = blockIdx.x;
  const int hk = lin % a.n_kv_heads;
  const int rest = lin / a.n_kv_heads;
  // Requests go in the caller's order (longest context first when it passes
  // one), each request's row blocks together so they share L2.
  const int ri = rest / a.row_blocks;
  const int bx = rest - ri * a.row_blocks;
  const int i = a.order ? a.order[ri] : ri;
  const int G = a.group;
  const int q0 = a.qo_indptr[i];
  const int q_len = a.qo_indptr[i + 1] - q0;
  const int kv_len = a.kv_indptr[i + 1] - a.kv_indptr[i];
  const int rows = q_len * G;
  const int nblk = (rows + BM - 1) / BM;
  if (bx >= nblk) return;
  const int rb = nblk - 1 - bx;  // heaviest row block first
  const int prefix = kv_len - q_len;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;

  // This lane's query row (column of S^T / O^T).
  const int r = rb * BM + wave * WROWS + col;
  const bool row_ok = r < rows;
  const int t = row_ok ? r / G : 0;
  const int g = row_ok ? r - t * G : 0;
  const int h = hk * G + g;
  // Keys visible to this row.
  const int lim = !row_ok ? 0 : (a.causal ? prefix + t + 1 : kv_len);

  // Keys any row of the workgroup sees, and the tiles every row sees whole.
  const int r_last = min(rows, (rb + 1) * BM) - 1;
  const int kv_end = a.causal ? min(kv_len, prefix + r_last / G + 1) : kv_len;
  const int ntiles = (kv_end + BN - 1) / BN;
  const int wg_min_lim = a.causal ? prefix + (rb * BM) / G + 1 : kv_len;
  const int n_free = min(ntiles, wg_min_lim / BN);

  // Q (B operand of S^T): lane holds dims 16s + 8*half .. +8 of its row for step s.
  uint4 qf[KSTEPS];
  {
    const uint16_t *qrow = reinterpret_cast<const uint16_t *>(a.q) +
                           ((int64_t)(q0 + t) * a.n_heads + h) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      qf[s] = row_ok ? load16(qrow + 16 * s) : make_uint4(0u, 0u, 0u, 0u);
  }

  const int32_t *table = a.req_to_token + (int64_t)a.req_pool_indices[i] * a.max_ctx_len;
  const uint32_t row_bytes = (uint32_t)a.n_kv_heads * D * 2;
  const char *kbase = reinterpret_cast<const char *>(a.k_layer) + (int64_t)hk * D * 2;
  const char *vbase = reinterpret_cast<const char *>(a.v_layer) + (int64_t)hk * D * 2;
  auto row_addr = [&](const char *base, int slot, uint32_t col_bytes) -> const char * {
    if constexpr (OFF32)
      return base + ((uint32_t)slot * row_bytes + col_bytes);
    else
      return base + ((int64_t)slot * row_bytes + col_bytes);
  };

  // Global -> register staging of one tile.  K: 16 lanes cover one key row.
  // V: lanes first run over the 16 key quads of the tile, so that the
  // transposed LDS writes of a 16-lane group fill 128 distinct bytes.
  // Two register stages (A, B) alternate, so rows are fetched two tiles
  // before they are staged into LDS.
  uint4 kregA[KPIECES], vregA[4], kregB[KPIECES], vregB[4];
  const int vkq = tid & 15;  // keys 4 * vkq .. + 3
  const int vdg = tid >> 4;  // dims 8 * vdg .. + 7
  const bool vjob = VJOBS >= NT || tid < VJOBS;  // compile-time true for head_dim 128

  // Slot ids are loaded one tile ahead of the rows they address, so a
  // tile's K/V loads never wait on a table load.  Keys past kv_end read the
  // last valid key instead (always masked), keeping every load unconditional.
  int kslot[KPIECES], vslot[4];
  auto slot_of = [&](int j) { return table[(uint32_t)min(j, kv_end - 1)]; };
  auto load_slots = [&](int tile) {
    const int base = tile * BN;
#pragma unroll
    for (int p = 0; p < KPIECES; ++p) kslot[p] = slot_of(base + (tid + NT * p) / (D / 8));
#pragma unroll
    for (int c = 0; c < 4; ++c) vslot[c] = slot_of(base + vkq * 4 + c);
  };
  auto fetch = [&](int tile, uint4(&kreg)[KPIECES], uint4(&vreg)[4]) {
#pragma unroll
    for (int p = 0; p < KPIECES; ++p) {
      const uint32_t dg = (tid + NT * p) % (D / 8);
      kreg[p] = load16(row_addr(kbase, kslot[p], dg * 16));
    }
    if (vjob) {
#pragma unroll
      for (int c = 0; c < 4; ++c) vreg[c] = load16(row_addr(vbase, vslot[c], vdg * 16));
    }
    load_slots(tile + 1);
  };

  auto stash = [&](Smem<D> &buf, const uint4(&kreg)[KPIECES], const uint4(&vreg)[4]) {
#pragma unroll
    for (int p = 0; p < KPIECES; ++p) {
      const int piece = tid + NT * p;
      const int key = piece / (D / 8);
      const int dg = piece - key * (D / 8);
      store16(&buf.k[key * KS + dg * 8], kreg[p]);
    }
    if (vjob) {
      // Transpose 4 keys x 8 dims: each dim becomes 4 contiguous keys.
      const int pos = vpos(vkq * 4);
      const uint32_t w[4][4] = {{vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w},
                                {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w},
                                {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w},
                                {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w}};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        uint2 v;
        v.x = __builtin_amdgcn_perm(w[1][e >> 1], w[0][e >> 1], sel);
        v.y = __builtin_amdgcn_perm(w[3][e >> 1], w[2][e >> 1], sel);
        *reinterpret_cast<uint2 *>(&buf.vt[(vdg * 8 + e) * VS + pos]) = v;
      }
    }
  };

  f32x16_t o[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int x = 0; x < 16; ++x) o[db][x] = 0.f;
  // Running max in raw score units (sm_scale > 0 keeps the order); this
  // lane's share of the running sum (its half of the keys).
  float m_run = kNegInf, l_lane = 0.f;
  const float c2 = a.scale_log2;
  const f32x16_t zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                           0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  constexpr uint32_t kOnes = 0x3f803f80u;  // bf16 pair (1, 1)

  // S^T of one 64-key tile (two 32-key blocks).
  auto qk = [&](const Smem<D> &buf, f32x16_t(&sacc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint16_t *krow = &buf.k[(kb * 32 + col) * KS + 8 * half];
      sacc[kb] = mfma32(*reinterpret_cast<const uint4 *>(krow), qf[0], zero16);
#pragma unroll
      for (int s = 1; s < KSTEPS; ++s)
        sacc[kb] = mfma32(*reinterpret_cast<const uint4 *>(krow + 16 * s), qf[s], sacc[kb]);
    }
  };

  // (Mask,) online softmax of one tile's S^T, then O^T += V^T P^T.
  auto softmax_pv = [&](int tile, f32x16_t(&sacc)[2], const Smem<D> &buf, auto masked) {
    constexpr bool MASK = decltype(masked)::value;
    if constexpr (MASK) {
      const int kbase_idx = tile * BN + 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int x = 0; x < 16; ++x)
          if (kbase_idx + kb * 32 + 8 * (x >> 2) + (x & 3) >= lim) sacc[kb][x] = kNegInf;
    }
    float tmax = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int x = 0; x < 16; ++x) tmax = fmaxf(tmax, sacc[kb][x]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    if (__any(m_new > m_run)) {  // rescale only when some row's max moved
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2((m_run - m_new) * c2);
      l_lane *= alpha;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) o[db] *= alpha;
      m_run = m_new;
    }
    const float mc = (m_run == kNegInf) ? 0.f : m_run * c2;
    // Per 16-key step: weights for those keys, rounded to bf16, then the PV
    // products that consume them.
#pragma unroll
    for (int ts = 0; ts < 4; ++ts) {
      const int kb = ts >> 1;
      const int x0 = 8 * (ts & 1);
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(sacc[kb][x0 + e], c2, -mc));
      uint4 pf;
      pf.x = pack_bf16x2(p[0], p[1]);
      pf.y = pack_bf16x2(p[2], p[3]);
      pf.z = pack_bf16x2(p[4], p[5]);
      pf.w = pack_bf16x2(p[6], p[7]);
      // the row sum uses the same bf16 weights the PV product sees
      l_lane = dot2_bf16(pf.x, kOnes, l_lane);
      l_lane = dot2_bf16(pf.y, kOnes, l_lane);
      l_lane = dot2_bf16(pf.z, kOnes, l_lane);
      l_lane = dot2_bf16(pf.w, kOnes, l_lane);
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const uint4 vf =
            *reinterpret_cast<const uint4 *>(&buf.vt[(db * 32 + col) * VS + 16 * ts + 8 * half]);
        o[db] = mfma32(vf, pf, o[db]);
      }
    }
  };

  // Pipeline, one barrier per tile: while tile n is multiplied from one LDS
  // buffer, the register stage holding tile n+1 is staged into the other
  // buffer and refilled with tile n+3; the other stage holds tile n+2 in
  // flight.  Tiles every row of the workgroup sees whole run an unmasked
  // step, the diagonal tiles a masked one (one code path per loop keeps the
  // register allocation tight).
  if (ntiles > 0) {
    load_slots(0);
    fetch(0, kregA, vregA);
    stash(sm[0], kregA, vregA);
    if (ntiles > 1) fetch(1, kregA, vregA);
    if (ntiles > 2) fetch(2, kregB, vregB);
    __syncthreads();
  }
  // The S^T products of tile n are issued first; the staging work for later
  // tiles (V transpose, LDS writes, row fetches) then runs on the vector and
  // memory units while the matrix cores work, followed by the softmax and PV
  // products.  Staging past the last tile writes an LDS buffer no tile reads
  // and reads clamped, valid rows: it is harmless and keeps the code
  // straight-line for the scheduler.
  auto step = [&](int tile, uint4(&kreg)[KPIECES], uint4(&vreg)[4], auto masked) {
    f32x16_t sacc[2];
    qk(sm[tile & 1], sacc);
    stash(sm[(tile + 1) & 1], kreg, vreg);
    fetch(tile + 3, kreg, vreg);
    softmax_pv(tile, sacc, sm[tile & 1], masked);
    __syncthreads();
  };
  const int n_free2 = n_free & ~1;
  int tile = 0;
  for (; tile < n_free2; tile += 2) {
    step(tile, kregA, vregA, std::false_type{});
    step(tile + 1, kregB, vregB, std::false_type{});
  }
  for (; tile + 1 < ntiles; tile += 2) {
    step(tile, kregA, vregA, std::true_type{});
    step(tile + 1, kregB, vregB, std::true_type{});
  }
  if (tile < ntiles) step(tile, kregA, vregA, std::true_type{});

  if (!row_ok) return;
  const float l_run = l_lane + __shfl_xor(l_lane, 32);
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  uint16_t *orow = reinterpret_cast<uint16_t *>(a.out) + ((int64_t)(q0 + t) * a.n_heads + h) * D;
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int x4 = 0; x4 < 4; ++x4) {
      const int d0 = db * 32 + 8 * x4 + 4 * half;
      uint2 w;
      w.x = pack_bf16x2(o[db][4 * x4 + 0] * inv, o[db][4 * x4 + 1] * inv);
      w.y = pack_bf16x2(o[db][4 * x4 + 2] * inv, o[db][4 * x4 + 3] * inv);
      *reinterpret_cast<uint2 *>(orow + d0) = w;
    }
}

}  // namespace

hipError_t launch_paged_prefill(const PrefillArgs &a, int head_dim, hipStream_t stream) {
  const int64_t row_blocks = ((int64_t)a.max_q_len * a.group + BM - 1) / BM;
  if (row_blocks > INT32_MAX) return hipErrorInvalidValue;
  const int64_t blocks = row_blocks * a.n_kv_heads * a.batch;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  PrefillArgs args = a;
  args.row_blocks = (int32_t)row_blocks;
  const dim3 grid((uint32_t)blocks);
  const uint64_t layer_bytes = (uint64_t)a.pool_size * a.n_kv_heads * head_dim * 2;
  const bool off32 = layer_bytes <= 0xffffffffull;
  if (head_dim == 128) {
    if (off32)
      hipLaunchKernelGGL((prefill_kernel<128, true>), grid, dim3(NT), 0, stream, args);
    else
      hipLaunchKernelGGL((prefill_kernel<128, false>), grid, dim3(NT), 0, stream, args);
  } else if (head_dim == 64) {
    if (off32)
      hipLaunchKernelGGL((prefill_kernel<64, true>), grid, dim3(NT), 0, stream, args);
    else
      hipLaunchKernelGGL((prefill_kernel<64, false>), grid, dim3(NT), 0, stream, args);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pkv

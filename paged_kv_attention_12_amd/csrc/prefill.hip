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
// Tiling.  A workgroup (8 wavefronts) owns one (request, kv-head, block of 256
// query rows), where the rows of a request enumerate (token t, head g of the
// kv-head's group) as r = t * G + g, so all G query heads sharing a kv-head
// reuse one K/V tile and any group size works.  Each wavefront owns 32 rows.
// Keys stream through LDS in tiles of 64, gathered by slot:
//   S^T (keys x rows) = K Q^T : v_mfma_f32_32x32x16_bf16, A = K rows from LDS,
//                               B = the wave's Q rows held in registers;
//   O^T (dims x rows) += V^T P^T : A = V^T, read from the V rows in LDS with
//                               transposing LDS reads (ds_read_b64_tr_b16),
//                               B = the softmax weights, rounded to bf16,
//                               taken straight from the S^T accumulators.
// With S^T in this orientation every lane holds one query row, so the
// online-softmax row max / row sum need one cross-lane step (lane l ^ 32).
//
// Schedule.  A SIMD holds two wavefronts of the workgroup, one from each of
// two groups (waves 0-3 and 4-7).  Both run the same tile pipeline, rotated
// by half a tile: while one is in its matrix-core phase (S^T products) the
// other is in its vector phase (softmax), so the two phases overlap on the
// SIMD instead of both waves waiting on the same unit.  One barrier per tile;
// tile n lives in LDS buffer n % 3 because the second group still reads tile
// n-1 while tile n+1 is being staged.
#include <math.h>

#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace pkv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kNegInf = -INFINITY;
constexpr int NT = 512;              // threads per workgroup (8 wavefronts)
constexpr int BN = 64;               // keys per tile
constexpr int WROWS = 32;            // query rows per wavefront
constexpr int BM = NT / 64 * WROWS;  // query rows per workgroup
static_assert(BM == kPrefillBlockRows, "row block size");
constexpr int NBUF = 3;              // LDS tile buffers
constexpr float kSlack = 8.f;        // log2 headroom before the running max is raised

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4 &v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ f32x16_t mfma32(const uint4 &a, const uint4 &b, const f32x16_t &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Workgroup barrier that orders LDS accesses only: the global loads in
// flight (rows fetched for later tiles) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// ds_read_b64_tr_b16: within each 16-lane group, lane j supplies the address
// of 4 consecutive 16-bit elements (row j of a 16 x 4 block M); lane l then
// receives M[l/4 + 4r][l%4] for r = 0..3.  With row j = (key j/4, dims
// 4(j%4) .. +3) of a [key][dim] tile, lane l receives dim l of 4 consecutive
// keys: the V^T operand read straight from V rows.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t *p) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p);
  return __builtin_bit_cast(uint2, v);
}

template <int DK, int DV>
struct Smem {
  static constexpr int KS = DK + 8;   // K row stride (elements), 16-byte pad
  static constexpr int VS = DV + 32;  // V row stride (elements), 64-byte pad
  uint16_t k[BN * KS];
  uint16_t v[BN * VS];
};

// Query rows of request i: its new tokens times the group size.
__device__ __forceinline__ int rows_of(const PrefillArgs &a, int i) {
  return (a.qo_indptr[i + 1] - a.qo_indptr[i]) * a.group;
}

// OFF32: every row of the layer lies within 4 GiB of the layer base, so row
// addresses are a uniform 64-bit base plus a 32-bit byte offset.  PAGED: the
// table holds page ids of pages of 2^page_shift tokens (else slot ids).  DK:
// width of the query and key rows; DV: of the value and output rows (MLA
// layers: keys qk_nope + qk_rope wide, values narrower).
template <int DK, int DV, bool OFF32, bool PAGED>
__global__ void __launch_bounds__(NT, 2) prefill_kernel(const PrefillArgs a) {
  using SM = Smem<DK, DV>;
  constexpr int KS = SM::KS;
  constexpr int VS = SM::VS;
  constexpr int KSTEPS = DK / 16;            // MFMA steps over the key width for S^T
  // K fragments of a 32-key block are read in runs of KRUN steps before
  // their products (all of them for keys up to 128 wide)
  constexpr int KRUN = KSTEPS > 8 ? 4 : KSTEPS;
  static_assert(KSTEPS % KRUN == 0, "fragment runs");
  constexpr int DBLK = DV / 32;              // 32-dim blocks of O^T
  constexpr int KPK = BN * DK / 8 / NT;      // 16-byte K pieces per thread per tile
  constexpr int KPV = BN * DV / 8 / NT;      // 16-byte V pieces per thread per tile
  constexpr bool SAME = DK == DV;            // then one slot id serves a K and a V piece
  constexpr int NSLOT = SAME ? KPK : KPK + KPV;
  static_assert(KPK >= 1 && KPV >= 1, "staging split");
  __shared__ SM sm[NBUF];

  // Workgroups are dispatched to the 8 XCDs round-robin by linear id; taking
  // the kv-head from the low part of the id keeps every workgroup of one
  // kv-head on the same XCD (for 8 kv-heads), so the row blocks of a request
  // share that head's K/V rows in one L2.
  const int lin = blockIdx.x;
  const int hk = lin % a.n_kv_heads;
  const int rest = lin / a.n_kv_heads;
  // Requests go in the caller's order (longest context first when it passes
  // one), each request's row blocks together so they share L2, the block of
  // the last rows (the most keys) first.  With a block list the launch holds
  // exactly the non-empty blocks in that order; without one it covers
  // row_blocks blocks of every request and the ones past its rows exit.
  int i, rb;
  if (a.blocks) {
    i = a.blocks[2 * rest];
    rb = a.blocks[2 * rest + 1];
  } else {
    const int ri = rest / a.row_blocks;
    const int bx = rest - ri * a.row_blocks;
    i = a.order ? a.order[ri] : ri;
    const int nblk = (rows_of(a, i) + BM - 1) / BM;
    if (bx >= nblk) return;
    rb = nblk - 1 - bx;
  }
  const int G = a.group;
  const int q0 = a.qo_indptr[i];
  const int q_len = a.qo_indptr[i + 1] - q0;
  const int kv_len = a.kv_indptr[i + 1] - a.kv_indptr[i];
  const int rows = q_len * G;
  const int prefix = kv_len - q_len;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int half = lane >> 5;
  const int col = lane & 31;

  // This lane's query row (column of S^T / O^T) and the keys it sees.
  const int r = rb * BM + wave * WROWS + col;
  const bool row_ok = r < rows;
  const int t = row_ok ? r / G : 0;
  const int h = hk * G + (row_ok ? r - t * G : 0);
  const int lim = !row_ok ? 0 : (a.causal ? prefix + t + 1 : kv_len);

  // Keys any row of the workgroup sees, and the tiles every row sees whole.
  // A workgroup that gets here has at least one row, so ntiles >= 1.
  const int r_last = min(rows, (rb + 1) * BM) - 1;
  const int kv_end = a.causal ? min(kv_len, prefix + r_last / G + 1) : kv_len;
  const int ntiles = (kv_end + BN - 1) / BN;
  const int wg_min_lim = a.causal ? prefix + (rb * BM) / G + 1 : kv_len;
  const int n_free = min(ntiles, wg_min_lim / BN);
  // Keys any row of this wavefront sees: in the tiles that need the mask, a
  // 32-key block at or past this limit is masked for all 32 rows, and its
  // products and weights are skipped.
  const int w_first = rb * BM + wave * WROWS;
  const int w_last = min(rows, w_first + WROWS) - 1;
  const int wave_lim = w_last < w_first ? 0 : (a.causal ? prefix + w_last / G + 1 : kv_len);

  // Q (B operand of S^T): lane holds dims 16s + 8*half .. +8 of its row for step s.
  uint4 qf[KSTEPS];
  {
    const uint16_t *qrow =
        reinterpret_cast<const uint16_t *>(a.q) + ((int64_t)(q0 + t) * a.n_heads + h) * DK + 8 * half;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      qf[s] = row_ok ? load16(qrow + 16 * s) : make_uint4(0u, 0u, 0u, 0u);
  }

  const int32_t *table = a.req_to_token + (int64_t)a.req_pool_indices[i] * a.table_stride;
  const uint32_t krow_bytes = (uint32_t)a.n_kv_heads * DK * 2;
  const uint32_t vrow_bytes = (uint32_t)a.n_kv_heads * DV * 2;
  const char *kbase = reinterpret_cast<const char *>(a.k_layer) + (int64_t)hk * DK * 2;
  const char *vbase = reinterpret_cast<const char *>(a.v_layer) + (int64_t)hk * DV * 2;
  auto row_addr = [&](const char *base, uint32_t row_bytes, int slot,
                      uint32_t col_bytes) -> const char * {
    if constexpr (OFF32)
      return base + ((uint32_t)slot * row_bytes + col_bytes);
    else
      return base + ((int64_t)slot * row_bytes + col_bytes);
  };

  // Global -> register staging of one tile: every thread copies KPK 16-byte
  // pieces of K and KPV of V (16 lanes per 128-dim row); with equal widths
  // one slot id serves a K and a V piece.
  uint4 kreg[KPK], vreg[KPV];

  // Slot ids are loaded one tile ahead of the rows they address, so a
  // tile's K/V loads never wait on a table load.  They are issued before the
  // rows of the current fetch: the memory counter drains in issue order, so
  // the next fetch's wait for its slot ids leaves these rows in flight.  Keys
  // past kv_end read the last valid key instead (always masked), keeping
  // every load unconditional.
  int slot[NSLOT];
  auto slot_of = [&](int j) {
    const uint32_t pos = (uint32_t)min(j, kv_end - 1);
    if constexpr (PAGED)
      return slot_of_pos(table, pos, a.page_shift);
    else
      return table[pos];
  };
  auto load_slots = [&](int tile, int(&ks)[NSLOT]) {
    const int base = tile * BN;
#pragma unroll
    for (int p = 0; p < KPK; ++p) ks[p] = slot_of(base + (tid + NT * p) / (DK / 8));
    if constexpr (!SAME) {
#pragma unroll
      for (int p = 0; p < KPV; ++p) ks[KPK + p] = slot_of(base + (tid + NT * p) / (DV / 8));
    }
  };
  auto fetch = [&](int tile) __attribute__((always_inline)) {
    int ns[NSLOT];
    load_slots(tile + 1, ns);
    __builtin_amdgcn_sched_barrier(0);  // keep the issue order: slot ids, then rows
#pragma unroll
    for (int p = 0; p < KPK; ++p) {
      const uint32_t dg = (tid + NT * p) % (DK / 8);
      kreg[p] = load16(row_addr(kbase, krow_bytes, slot[p], dg * 16));
      if constexpr (SAME) vreg[p] = load16(row_addr(vbase, vrow_bytes, slot[p], dg * 16));
    }
    if constexpr (!SAME) {
#pragma unroll
      for (int p = 0; p < KPV; ++p) {
        const uint32_t dg = (tid + NT * p) % (DV / 8);
        vreg[p] = load16(row_addr(vbase, vrow_bytes, slot[KPK + p], dg * 16));
      }
    }
#pragma unroll
    for (int p = 0; p < NSLOT; ++p) slot[p] = ns[p];
  };

  auto stash = [&](SM &buf) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < KPK; ++p) {
      const int piece = tid + NT * p;
      const int key = piece / (DK / 8);
      const int dg = piece - key * (DK / 8);
      store16(&buf.k[key * KS + dg * 8], kreg[p]);
    }
#pragma unroll
    for (int p = 0; p < KPV; ++p) {
      const int piece = tid + NT * p;
      const int key = piece / (DV / 8);
      const int dg = piece - key * (DV / 8);
      store16(&buf.v[key * VS + dg * 8], vreg[p]);
    }
  };

  f32x16_t o[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int x = 0; x < 16; ++x) o[db][x] = 0.f;
  // Running max in raw score units (sm_scale > 0 keeps the order), the raw
  // score above which it must move, and this lane's share of the running sum
  // (its half of the keys).
  // Transposed V reads: lane l of 16-lane group g addresses key (l%16)/4 of
  // its 4-key run, dims 16(g&1) + 4(l%4) .. +3 of the 32-dim block.
  const int gl = lane & 15;
  const int voff = 16 * ((lane >> 4) & 1) + 4 * (gl & 3);
  const float c2 = a.scale_log2;
  const float slack_raw = kSlack / c2;
  float m_run = kNegInf, m_thr = kNegInf, l_lane = 0.f;
  const f32x16_t zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                           0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  constexpr uint32_t kOnes = 0x3f803f80u;  // bf16 pair (1, 1)

  // S^T of one 64-key tile (two 32-key blocks).  All fragment reads of a
  // block are issued before its products, so the products do not wait on
  // LDS latency one read at a time.  In a tile that needs the mask, a block
  // past every row of the wavefront is set to -inf without its products.
  const f32x16_t ninf16 = {kNegInf, kNegInf, kNegInf, kNegInf, kNegInf, kNegInf, kNegInf, kNegInf,
                           kNegInf, kNegInf, kNegInf, kNegInf, kNegInf, kNegInf, kNegInf, kNegInf};
  auto qk = [&](const SM &buf, f32x16_t(&sacc)[2], int tile,
                auto masked) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(masked)::value;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (MASK && tile * BN + 32 * kb >= wave_lim) {
        sacc[kb] = ninf16;  // every key of the block is past every row of this wave
        continue;
      }
      const uint16_t *krow = &buf.k[(kb * 32 + col) * KS + 8 * half];
#pragma unroll
      for (int r0 = 0; r0 < KSTEPS; r0 += KRUN) {
        uint4 kf[KRUN];
#pragma unroll
        for (int s = 0; s < KRUN; ++s)
          kf[s] = *reinterpret_cast<const uint4 *>(krow + 16 * (r0 + s));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < KRUN; ++s)
          sacc[kb] = mfma32(kf[s], qf[r0 + s], r0 + s == 0 ? zero16 : sacc[kb]);
      }
    }
  };

  // (Mask,) online softmax of one tile's S^T, then O^T += V^T P^T.
  auto softmax_pv = [&](int tile, f32x16_t(&sacc)[2], const SM &buf,
                        auto masked) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(masked)::value;
    if constexpr (MASK) {
      const int kbase_idx = tile * BN + 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int x = 0; x < 16; ++x)
          if (kbase_idx + kb * 32 + 8 * (x >> 2) + (x & 3) >= lim) sacc[kb][x] = kNegInf;
    }
    // Max over this lane's half of the row (32 of the tile's 64 keys): a
    // tree of three-input maxes, 17 instructions at depth 4.
    auto max3 = [](float x, float y, float z) { return fmaxf(fmaxf(x, y), z); };
    float m11[11];
#pragma unroll
    for (int j = 0; j < 10; ++j) {
      const int e = 3 * j;
      m11[j] = max3(sacc[e >> 4][e & 15], sacc[(e + 1) >> 4][(e + 1) & 15],
                    sacc[(e + 2) >> 4][(e + 2) & 15]);
    }
    m11[10] = fmaxf(sacc[1][14], sacc[1][15]);
    const float tmax = fmaxf(max3(max3(m11[0], m11[1], m11[2]), max3(m11[3], m11[4], m11[5]),
                                  max3(m11[6], m11[7], m11[8])),
                             fmaxf(m11[9], m11[10]));
    // The reference max only moves when a score exceeds it by more than
    // 2^kSlack in weight; below that, weights up to 2^kSlack accumulate
    // against the old reference (exact: numerator and denominator share it),
    // so the O rescale is rare after the first tiles.  Each half of the wave
    // tests its own keys; only a move needs the row max over both halves.
    if (__any(tmax > m_thr)) {
      const float m_new = fmaxf(m_run, fmaxf(tmax, __shfl_xor(tmax, 32)));
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2((m_run - m_new) * c2);
      l_lane *= alpha;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) o[db] *= alpha;
      m_run = m_new;
      m_thr = m_new + slack_raw;
    }
    const float mc = (m_run == kNegInf) ? 0.f : m_run * c2;
    // Per 16-key step: weights for those keys, rounded to bf16, then the PV
    // products that consume them.
#pragma unroll
    for (int ts = 0; ts < 4; ++ts) {
      const int kb = ts >> 1;
      const int x0 = 8 * (ts & 1);
      if (MASK && tile * BN + 32 * kb >= wave_lim) continue;  // weights all 0
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
        // V^T operand: keys 16ts + 4half + {0..3} and 16ts + 8 + 4half + {0..3}
        // (the keys this lane's weights cover), dim db*32 + lane % 32.
        const uint16_t *vb = &buf.v[(16 * ts + 4 * half + (gl >> 2)) * VS + db * 32 + voff];
        const uint2 lo = lds_read_tr16(vb);
        const uint2 hi = lds_read_tr16(vb + 8 * VS);
        o[db] = mfma32(make_uint4(lo.x, lo.y, hi.x, hi.y), pf, o[db]);
      }
    }
  };

  // Prologue: tile 0 in buffer 0, tile 1 in registers.  It is unconditional
  // (fetches past the last tile read clamped, valid rows), so every path into
  // the tile loops has waited for the Q loads and the loops' memory waits
  // stay exact.
  load_slots(0, slot);
  fetch(0);
  stash(sm[0]);
  fetch(1);
  __syncthreads();

  // Period k (between two barriers): tile k+1 goes from registers to LDS,
  // tile k+2 is fetched.  The first group multiplies S^T(k) and then does
  // softmax / PV of tile k; the second group first finishes tile k-1
  // (softmax / PV) and then multiplies S^T(k).  Staging past the last tile
  // writes a buffer no tile reads and reads clamped, valid rows.  Tiles every
  // row of the workgroup sees whole skip the mask (separate loops keep the
  // register allocation of each tight).  Both groups pass the same number of
  // barriers.
  f32x16_t sacc[2];
  int cur = 0;   // buffer of tile k
  int prev = 2;  // buffer of tile k-1
  auto next_buf = [](int b) { return b == NBUF - 1 ? 0 : b + 1; };
  if (wave < 4) {
    auto period = [&](int k, auto masked) __attribute__((always_inline)) {
      const int nb = next_buf(cur);
      qk(sm[cur], sacc, k, masked);
      stash(sm[nb]);
      fetch(k + 2);
      softmax_pv(k, sacc, sm[cur], masked);
      lds_barrier();
      cur = nb;
    };
    int k = 0;
    for (; k < n_free; ++k) period(k, std::false_type{});
    for (; k < ntiles; ++k) period(k, std::true_type{});
  } else {
    auto period = [&](int k, auto masked) __attribute__((always_inline)) {
      const int nb = next_buf(cur);
      // tile k-1 < k: the mask choice made for tile k is safe for it
      softmax_pv(k - 1, sacc, sm[prev], masked);
      stash(sm[nb]);
      fetch(k + 2);
      qk(sm[cur], sacc, k, masked);
      lds_barrier();
      prev = cur;
      cur = nb;
    };
    // period 0: no earlier tile to finish
    stash(sm[1]);
    fetch(2);
    if (n_free > 0)
      qk(sm[0], sacc, 0, std::false_type{});
    else
      qk(sm[0], sacc, 0, std::true_type{});
    lds_barrier();
    prev = 0;
    cur = 1;
    int k = 1;
    for (; k < n_free; ++k) period(k, std::false_type{});
    for (; k < ntiles; ++k) period(k, std::true_type{});
    softmax_pv(ntiles - 1, sacc, sm[prev], std::true_type{});
  }

  const float l_run = l_lane + __shfl_xor(l_lane, 32);
  if (!row_ok) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  uint16_t *orow = reinterpret_cast<uint16_t *>(a.out) + ((int64_t)(q0 + t) * a.n_heads + h) * DV;
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

template <int DK, int DV>
hipError_t launch_d(const PrefillArgs &a, bool off32, hipStream_t stream) {
  const int64_t row_blocks = ((int64_t)a.max_q_len * a.group + BM - 1) / BM;
  if (row_blocks > INT32_MAX) return hipErrorInvalidValue;
  const int64_t blocks = (a.blocks ? a.n_blocks : row_blocks * a.batch) * a.n_kv_heads;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  PrefillArgs args = a;
  args.row_blocks = (int32_t)row_blocks;
  const dim3 grid((uint32_t)blocks);
  const bool paged = a.page_shift > 0;
  if (off32 && !paged)
    hipLaunchKernelGGL((prefill_kernel<DK, DV, true, false>), grid, dim3(NT), 0, stream, args);
  else if (off32)
    hipLaunchKernelGGL((prefill_kernel<DK, DV, true, true>), grid, dim3(NT), 0, stream, args);
  else if (!paged)
    hipLaunchKernelGGL((prefill_kernel<DK, DV, false, false>), grid, dim3(NT), 0, stream, args);
  else
    hipLaunchKernelGGL((prefill_kernel<DK, DV, false, true>), grid, dim3(NT), 0, stream, args);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_paged_prefill(const PrefillArgs &a, int head_dim, int v_head_dim,
                                hipStream_t stream) {
  // Offsets fit 32 bits when the wider (key) rows of the whole layer do.
  const uint64_t layer_bytes = (uint64_t)a.pool_size * a.n_kv_heads * head_dim * 2;
  const bool off32 = layer_bytes <= 0xffffffffull;
  if (head_dim == 128 && v_head_dim == 128) return launch_d<128, 128>(a, off32, stream);
  if (head_dim == 64 && v_head_dim == 64) return launch_d<64, 64>(a, off32, stream);
  if (head_dim == 192 && v_head_dim == 128) return launch_d<192, 128>(a, off32, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv

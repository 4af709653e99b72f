// Device-side helpers shared by the libpkv kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// bf16 values are carried as raw 16-bit patterns; two of them share a dword.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bit pattern, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two fp32 -> one dword of two bf16 (lo in bits 0..15), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// a.lo*b.lo + a.hi*b.hi + c with bf16 pairs held in dwords (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// 2^x on the transcendental unit; 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane permutations inside a row of 16 lanes.
enum : int {
  DPP_QUAD_XOR1 = 0xB1,      // quad_perm [1,0,3,2]
  DPP_QUAD_XOR2 = 0x4E,      // quad_perm [2,3,0,1]
  DPP_ROW_MIRROR = 0x140,    // lane i <- lane 15-i
  DPP_ROW_HALF_MIRROR = 0x141  // lane i <- lane 7-i within each half row
};

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N in {4, 8, 16, 32, 64}); every lane of
// a group receives the group total.  Groups up to 16 use DPP only.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
  x += dpp_f32<DPP_QUAD_XOR1>(x);
  x += dpp_f32<DPP_QUAD_XOR2>(x);
  if constexpr (N >= 8) x += dpp_f32<DPP_ROW_HALF_MIRROR>(x);
  if constexpr (N >= 16) x += dpp_f32<DPP_ROW_MIRROR>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Slot of logical position j of a request whose table row is `row`: with
// pages of 2^page_shift tokens, entry j >> page_shift is the physical page and
// the position sits at offset j mod 2^page_shift of it (page_shift 0: the row
// holds slots).
__device__ __forceinline__ int32_t slot_of_pos(const int32_t *row, uint32_t j, int page_shift) {
  const uint32_t page = (uint32_t)row[j >> page_shift];
  return (int32_t)((page << page_shift) | (j & ((1u << page_shift) - 1u)));
}

// Rotary turn of one 16-byte piece of a bf16 row: pairs (a, b) = elements
// (2j, 2j+1) times (c + i s) = (cs[2j], cs[2j+1]), in fp32, rounded to bf16.
// The same arithmetic as the rotary kernel's, so a row turned here equals
// the row that kernel writes, bit for bit.
__device__ __forceinline__ uint4 rotate_bf16x8(const uint4 &w, const float *cs) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  uint32_t r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = bf16_lo(u[j]), b = bf16_hi(u[j]);
    const float c = cs[2 * j], s = cs[2 * j + 1];
    r[j] = pack_bf16x2(fmaf(a, c, -(b * s)), fmaf(a, s, b * c));
  }
  return make_uint4(r[0], r[1], r[2], r[3]);
}

__device__ __forceinline__ uint4 load16(const void *p) {
  return *reinterpret_cast<const uint4 *>(p);
}
// A 16-byte load with the non-temporal hint (global_load_dwordx4 ... nt):
// for rows read once, so that they do not displace lines read again.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_nt(const void *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store16(void *p, uint4 v) {
  *reinterpret_cast<uint4 *>(p) = v;
}

}  // namespace pkv

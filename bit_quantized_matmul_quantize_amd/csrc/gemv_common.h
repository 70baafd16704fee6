// Device helpers shared by the bandwidth-bound GEMV kernels (Q2_0 and Q4_K):
// bf16 pair dot products, constant masks in VGPRs, the activation pair
// permutation and DPP row/half-wave sums.
#pragma once

#include "bqmm_internal.h"

namespace bqmm {
namespace {

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, a), __builtin_bit_cast(v2bf, b), c, false);
}

__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t bits) {
  return (x & mask) | bits;
}

// A constant materialized in a VGPR and opaque to the optimizer.  gfx9 VOP3
// encodings take no literal, so with literal masks the compiler splits
// (x & m) | b into v_and_b32 + v_or_b32; with the masks in VGPRs it selects
// one v_and_or_b32 per code pair.
__device__ __forceinline__ uint32_t vconst(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

// Activation pairs of 16 consecutive values a[0..15] (eight bf16x2 words D):
// word i of the chunk pairs (4i, 4i+2) and (4i+1, 4i+3).
__device__ __forceinline__ void act_pairs(const uint32_t D[8], uint32_t p[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[2 * i] = __builtin_amdgcn_perm(D[2 * i + 1], D[2 * i], 0x05040100u);
    p[2 * i + 1] = __builtin_amdgcn_perm(D[2 * i + 1], D[2 * i], 0x07060302u);
  }
}

// x plus the value DPP moves into this lane (rows not in row_mask add 0).
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_add(float x) {
  const int moved = __builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, kRowMask, 0xF, false);
  return x + __int_as_float(moved);
}

// Sum over each group of 16 lanes; every lane of the group gets the total.
__device__ __forceinline__ float row16_sum(float x) {
  x = dpp_add<0xB1, 0xF>(x);   // quad_perm [1,0,3,2]: xor 1
  x = dpp_add<0x4E, 0xF>(x);   // quad_perm [2,3,0,1]: xor 2
  x = dpp_add<0x124, 0xF>(x);  // row_ror:4
  x = dpp_add<0x128, 0xF>(x);  // row_ror:8
  return x;
}

// Sum over each half-wave (lanes 0..31, 32..63); the total lands in lanes
// 16..31 and 48..63.
__device__ __forceinline__ float half_wave_sum(float x) {
  x = row16_sum(x);
  x = dpp_add<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
  return x;
}

}  // namespace
}  // namespace bqmm

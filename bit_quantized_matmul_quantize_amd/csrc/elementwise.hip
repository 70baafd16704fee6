// Bandwidth-bound elementwise kernels: Q2_0 -> bf16 dequant and silu_mul.
#include "bqmm_internal.h"

namespace bqmm {
namespace {

// Q2_0 -> bf16.  [page layers/qwen3_ssm/init_q2.rs, fn qkvz_q2_prefill_gemm,
// fallback branch: dequant_q2_0_gn_to_bf16(w, scratch, n, k, group).]
// One lane per 32-bit word of codes (16 weights).  The word holds bytes
// t0..t0+3 of a group, and field j of those bytes is the four consecutive
// weights at k-offsets j*G/4 + t0 .. +3, so every field becomes one 8-byte
// store.  Each group has only four values, d*(c-2) for c = 0..3; they are
// rounded once to bf16 and selected by code.  Reads 2.125 bits, writes 16 bits
// per weight.
__global__ __launch_bounds__(256) void dequant_q2_0_kernel(const uint8_t *__restrict__ w,
                                                           uint16_t *__restrict__ out, uint32_t n,
                                                           uint32_t k, uint32_t group) {
  // One lane per 8 code bytes (two words, always inside one group since
  // group % 32 == 0): field j of those bytes is 8 consecutive k, written as
  // one 16-byte store.
  const uint64_t pairs_per_row = k / 32u;
  const uint64_t total = (uint64_t)n * pairs_per_row;
  const uint32_t pairs_per_group = group / 32u;
  const uint16_t *scales = reinterpret_cast<const uint16_t *>(w + (uint64_t)n * k / 4u);
  const uint32_t groups_per_row = k / group;
  for (uint64_t pi = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; pi < total;
       pi += (uint64_t)gridDim.x * blockDim.x) {
    const uint64_t r = pi / pairs_per_row;
    const uint32_t pr = (uint32_t)(pi - r * pairs_per_row);
    const uint32_t g = pr / pairs_per_group;
    const uint32_t t0 = (pr - g * pairs_per_group) * 8u;
    const uint2 words = reinterpret_cast<const uint2 *>(w)[pi];
    const float d = f16_bits_to_f32(scales[r * groups_per_row + g]);
    const uint64_t lut = (uint64_t)f32_to_bf16_rne(-2.0f * d) |
                         ((uint64_t)f32_to_bf16_rne(-d) << 16) |
                         ((uint64_t)f32_to_bf16_rne(0.0f * d) << 32) |
                         ((uint64_t)f32_to_bf16_rne(d) << 48);
    uint16_t *dst = out + r * k + (uint64_t)g * group + t0;
#pragma unroll
    for (uint32_t j = 0; j < 4; ++j) {
      uint32_t v[8];
#pragma unroll
      for (uint32_t i = 0; i < 8; ++i) {
        const uint32_t c = (((i < 4) ? words.x : words.y) >> (8u * (i & 3u) + 2u * j)) & 3u;
        v[i] = (uint32_t)(lut >> (16u * c)) & 0xFFFFu;
      }
      *reinterpret_cast<uint4 *>(dst + j * (group / 4u)) =
          make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
    }
  }
}

// out = bf16(silu(gate) * up), silu(g) = g / (1 + exp(-g)) in binary32.
// [page layers/dense_ffn_decode_batch.rs, fn forward_km_q2: silu_mul over
//  m * intermediate elements, output over the gate buffer.]  Eight elements
// per lane; every lane reads its own elements before writing them, so
// out == gate is safe.
__global__ __launch_bounds__(256) void silu_mul_kernel(const uint16_t *gate, const uint16_t *up,
                                                       uint16_t *out, uint64_t count, int vec_ok) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x * 8u;
  for (uint64_t i0 = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8u; i0 < count;
       i0 += stride) {
    if (vec_ok && i0 + 8u <= count) {
      const uint4 gv = *reinterpret_cast<const uint4 *>(gate + i0);
      const uint4 uv = *reinterpret_cast<const uint4 *>(up + i0);
      const uint32_t ga[4] = {gv.x, gv.y, gv.z, gv.w};
      const uint32_t ua[4] = {uv.x, uv.y, uv.z, uv.w};
      uint32_t o[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float lo = silu_mul_f32(__uint_as_float(ga[t] << 16), __uint_as_float(ua[t] << 16));
        const float hi = silu_mul_f32(__uint_as_float(ga[t] & 0xFFFF0000u),
                                      __uint_as_float(ua[t] & 0xFFFF0000u));
        o[t] = pack_bf16x2(lo, hi);
      }
      *reinterpret_cast<uint4 *>(out + i0) = make_uint4(o[0], o[1], o[2], o[3]);
    } else {
      for (uint64_t i = i0; i < count && i < i0 + 8u; ++i)
        out[i] = (uint16_t)f32_to_bf16_rne(silu_mul_f32(bf16_to_f32(gate[i]), bf16_to_f32(up[i])));
    }
  }
}

uint32_t grid_for(uint64_t items, uint32_t per_block) {
  uint64_t b = (items + per_block - 1) / per_block;
  const uint64_t cap = 256u * 64u;  // enough waves to fill 256 CUs; the kernels stride
  if (b > cap) b = cap;
  if (b == 0) b = 1;
  return (uint32_t)b;
}

}  // namespace

hipError_t launch_dequant_q2_0(const void *w, void *out, uint32_t n, uint32_t k, uint32_t group,
                               hipStream_t s) {
  const uint64_t pairs = (uint64_t)n * (k / 32u);
  hipLaunchKernelGGL(dequant_q2_0_kernel, dim3(grid_for(pairs, 256)), dim3(256), 0, s,
                     static_cast<const uint8_t *>(w), static_cast<uint16_t *>(out), n, k, group);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const void *gate, const void *up, void *out, uint64_t count,
                           hipStream_t s) {
  const int vec_ok = ((reinterpret_cast<uintptr_t>(gate) | reinterpret_cast<uintptr_t>(up) |
                       reinterpret_cast<uintptr_t>(out)) & 15u) == 0u;
  hipLaunchKernelGGL(silu_mul_kernel, dim3(grid_for((count + 7) / 8, 256)), dim3(256), 0, s,
                     static_cast<const uint16_t *>(gate), static_cast<const uint16_t *>(up),
                     static_cast<uint16_t *>(out), count, vec_ok);
  return hipGetLastError();
}

}  // namespace bqmm

// bf16 activations -> q8_1 (blocks of 32 int8 codes with fp16 scale d and
// fp16 sum s).
//
// [page layers/ops/q4k_mmq.rs, fn quantize_act_q8_1: bf16 [m, k] in, q8_1 out,
//  k padded to 256.]  The page launches one 128-thread block per (row, 512
// values); here a 256-thread workgroup covers 2048 values of one row and each
// lane owns 8 consecutive values (one 16-byte load), so a 32-value block is
// four adjacent lanes and its max and sum are two butterfly steps.  Bandwidth
// bound: 2 bytes read and 1.125 bytes written per value.
//
// Rule (bit-exact contract): d = fp16_rne(amax / 127) with binary32
// division; q = clamp(roundf(x / float(d)), -127, 127) with binary32 division
// and ties away from zero; s = fp16_rne(float(d) * sum q).  A zero d gives zero
// codes.  Padding (k <= index < kpad) quantizes zeros.
//
// With kSiluMul the kernel quantizes the FFN's hidden activation straight
// from its producer: x = bf16_rne(silu(gate) * up) from two bf16 inputs, the
// value silu_mul_bf16 would store, so the bf16 tensor is never written.
#include "bqmm_internal.h"

namespace bqmm {
namespace {

constexpr int kThreads = 256;
constexpr int kPerLane = 8;
constexpr int kPerBlock = kThreads * kPerLane;  // values per workgroup

__device__ __forceinline__ float silu_mul_bf16_value(uint32_t g_bits16, uint32_t u_bits16) {
  return bf16_to_f32(f32_to_bf16_rne(silu_mul_f32(bf16_to_f32(g_bits16), bf16_to_f32(u_bits16))));
}

template <bool kSiluMul>
__global__ __launch_bounds__(kThreads) void quantize_q8_1_kernel(
    const uint16_t *__restrict__ act, const uint16_t *__restrict__ up, uint8_t *__restrict__ out,
    uint32_t k, uint32_t kpad, uint32_t chunks, uint64_t ds_offset, int vec_ok) {
  const uint32_t row = blockIdx.x / chunks;
  const uint32_t chunk = blockIdx.x - row * chunks;
  const uint32_t k0 = chunk * kPerBlock + threadIdx.x * kPerLane;
  // kpad is a multiple of 256, so the four lanes of a 32-block leave together.
  if (k0 >= kpad) return;

  const uint16_t *src = act + (uint64_t)row * k;
  const uint16_t *usrc = kSiluMul ? up + (uint64_t)row * k : nullptr;
  float x[kPerLane];
  if (vec_ok && k0 + kPerLane <= k) {
    const uint4 v = *reinterpret_cast<const uint4 *>(src + k0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if constexpr (kSiluMul) {
      const uint4 uv = *reinterpret_cast<const uint4 *>(usrc + k0);
      const uint32_t u[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = silu_mul_bf16_value(w[i] & 0xFFFFu, u[i] & 0xFFFFu);
        x[2 * i + 1] = silu_mul_bf16_value(w[i] >> 16, u[i] >> 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      if constexpr (kSiluMul)
        x[i] = (k0 + i < k) ? silu_mul_bf16_value(src[k0 + i], usrc[k0 + i]) : 0.0f;
      else
        x[i] = (k0 + i < k) ? bf16_to_f32(src[k0 + i]) : 0.0f;
    }
  }

  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));

  const uint32_t dh = f32_to_f16_bits(amax / 127.0f);
  const float d = f16_bits_to_f32(dh);

  int sum = 0;
  uint32_t packed[2] = {0u, 0u};
  if (d != 0.0f) {
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      float t = roundf(x[i] / d);
      t = fminf(fmaxf(t, -127.0f), 127.0f);
      const int q = (int)t;
      sum += q;
      packed[i / 4] |= ((uint32_t)q & 0xFFu) << (8 * (i % 4));
    }
  }
  sum += __shfl_xor(sum, 1);
  sum += __shfl_xor(sum, 2);

  *reinterpret_cast<uint2 *>(out + (uint64_t)row * kpad + k0) = make_uint2(packed[0], packed[1]);
  if ((threadIdx.x & 3u) == 0u) {
    const uint32_t sh = f32_to_f16_bits(d * (float)sum);
    const uint32_t pair = dh | (sh << 16);
    *reinterpret_cast<uint32_t *>(out + ds_offset + 4ull * ((uint64_t)row * (kpad / 32) + k0 / 32)) = pair;
  }
}

template <bool kSiluMul>
hipError_t launch_quantize(const void *act, const void *up, void *out, uint32_t m, uint32_t k,
                           hipStream_t s) {
  const uint32_t kpad = (k + 255u) / 256u * 256u;
  const uint32_t chunks = (kpad + kPerBlock - 1) / kPerBlock;
  const uint64_t blocks = (uint64_t)m * chunks;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(act) | reinterpret_cast<uintptr_t>(up);
  const int vec_ok = (k % 8u == 0u) && ((addr & 15u) == 0u);
  hipLaunchKernelGGL(quantize_q8_1_kernel<kSiluMul>, dim3((uint32_t)blocks), dim3(kThreads), 0, s,
                     static_cast<const uint16_t *>(act), static_cast<const uint16_t *>(up),
                     static_cast<uint8_t *>(out), k, kpad, chunks, (uint64_t)m * kpad, vec_ok);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_act_q8_1(const void *act, void *out, uint32_t m, uint32_t k,
                                    hipStream_t s) {
  return launch_quantize<false>(act, nullptr, out, m, k, s);
}

hipError_t launch_silu_mul_quantize_q8_1(const void *gate, const void *up, void *out, uint32_t m,
                                         uint32_t k, hipStream_t s) {
  return launch_quantize<true>(gate, up, out, m, k, s);
}

}  // namespace bqmm

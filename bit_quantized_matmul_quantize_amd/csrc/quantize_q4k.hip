// bf16 weights [n][k] -> block_q4_K [n][k/256] (256 weights in 144 bytes).
//
// [page layers/ops/q4k_mmq.rs, fn quantize_weight_q4k: bf16 [nrows,
//  n_per_row] to block_q4_K, one 256-value block per thread; the module
//  converts each weight once and caches it.]
//
// The page prints no rule; the one implemented (bit-exact contract, binary32
// with IEEE division and roundf) is an affine min/max fit per 32-value
// sub-block j whose step and offset are stored as 6-bit multiples of two fp16
// super-block scales:
//   lo_j = min(+0, min x), hi_j = max(lo_j, max x)
//   S_j = (hi_j - lo_j) / 15, M_j = 0 - lo_j
//   d = fp16_rne(max_j S_j / 63), dmin = fp16_rne(max_j M_j / 63)
//   sc_j = d > 0 ? min(63, roundf(S_j / d)) : 0; m_j likewise from M_j, dmin
//   q = clamp(roundf((x + dmin m_j) / (d sc_j)), 0, 15), 0 when d sc_j = 0.
// Both products are exact in binary32, so a fused multiply-add of the offset
// rounds the same sum.  Every candidate of a maximum is >= +0 and never -0,
// so the maxima do not depend on the reduction order.
//
// Layout: one wave per 8 super-blocks, one lane per sub-block.  A lane reads
// its 32 values (64 contiguous bytes), the group of 8 lanes reduces the two
// maxima and ORs the twelve scale/min bytes together with xor shuffles, and
// code bytes are formed by pairing lanes 2t (low nibbles) and 2t + 1 (high
// nibbles) of chunk t: each sends the other the half it needs and writes
// 16 of the chunk's 32 bytes.  Lane 0 of the group writes the 16-byte header.
#include "bqmm_internal.h"

namespace bqmm {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t code_of(float x, float off, float step) {
  if (!(step > 0.0f)) return 0u;
  const float t = roundf((x + off) / step);
  return t < 0.0f ? 0u : (t > 15.0f ? 15u : (uint32_t)t);
}

__device__ __forceinline__ uint32_t six_bits(float v, float scale) {
  if (!(scale > 0.0f)) return 0u;
  const float t = roundf(v / scale);
  return t > 63.0f ? 63u : (uint32_t)t;
}

__global__ __launch_bounds__(kThreads) void quantize_weight_q4k_kernel(const uint16_t *__restrict__ wb,
                                                                       uint8_t *__restrict__ out,
                                                                       uint64_t total_sb) {
  const uint64_t gid = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  const uint64_t sb = gid >> 3;
  const uint32_t j = threadIdx.x & 7u;
  // lanes past the last super-block compute on it (clamped) and store nothing
  const uint64_t sbl = sb < total_sb ? sb : total_sb - 1u;
  const uint4 *src = reinterpret_cast<const uint4 *>(wb + sbl * 256u + 32u * j);
  float x[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = src[q];
    const uint32_t words[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[8 * q + 2 * i] = bf16_to_f32(words[i] & 0xFFFFu);
      x[8 * q + 2 * i + 1] = bf16_to_f32(words[i] >> 16);
    }
  }
  float lo = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) lo = x[i] < lo ? x[i] : lo;
  float hi = lo;
#pragma unroll
  for (int i = 0; i < 32; ++i) hi = x[i] > hi ? x[i] : hi;
  const float S = (hi - lo) / 15.0f, M = 0.0f - lo;

  float maxS = S, maxM = M;
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    const float s2 = __shfl_xor(maxS, o, 8), m2 = __shfl_xor(maxM, o, 8);
    maxS = s2 > maxS ? s2 : maxS;
    maxM = m2 > maxM ? m2 : maxM;
  }
  const uint32_t dh = f32_to_f16_bits(maxS / 63.0f), mh = f32_to_f16_bits(maxM / 63.0f);
  const float d = f16_bits_to_f32(dh), dmin = f16_bits_to_f32(mh);
  const uint32_t sc = six_bits(S, d), mn = six_bits(M, dmin);
  const float step = d * (float)sc, off = dmin * (float)mn;

  // codes as bytes: wa = values 0..15, wb = values 16..31 of the sub-block
  uint32_t wa[4], wbv[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    wa[w] = code_of(x[4 * w], off, step) | (code_of(x[4 * w + 1], off, step) << 8) |
            (code_of(x[4 * w + 2], off, step) << 16) | (code_of(x[4 * w + 3], off, step) << 24);
    wbv[w] = code_of(x[16 + 4 * w], off, step) | (code_of(x[16 + 4 * w + 1], off, step) << 8) |
             (code_of(x[16 + 4 * w + 2], off, step) << 16) | (code_of(x[16 + 4 * w + 3], off, step) << 24);
  }
  // even lane (sub-block 2t, low nibbles) writes chunk bytes 0..15 and needs
  // the odd lane's values 0..15; the odd lane writes bytes 16..31.
  const bool odd = (j & 1u) != 0u;
  uint32_t outw[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t recv = (uint32_t)__shfl_xor((int)(odd ? wa[w] : wbv[w]), 1, 8);
    outw[w] = odd ? (recv | (wbv[w] << 4)) : (wa[w] | (recv << 4));
  }

  // scale/min bytes: j < 4 owns the low six bits of S[j] and S[j+4]; j >= 4
  // the top two bits of S[j-4] and S[j] and both nibbles of S[j+4]
  const uint32_t jj = j & 3u, sh = 8u * jj;
  uint32_t y, z, wq;
  if (j < 4u) {
    y = (sc & 63u) << sh;
    z = (mn & 63u) << sh;
    wq = 0u;
  } else {
    y = ((sc >> 4) << 6) << sh;
    z = ((mn >> 4) << 6) << sh;
    wq = ((sc & 15u) | ((mn & 15u) << 4)) << sh;
  }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    y |= (uint32_t)__shfl_xor((int)y, o, 8);
    z |= (uint32_t)__shfl_xor((int)z, o, 8);
    wq |= (uint32_t)__shfl_xor((int)wq, o, 8);
  }

  if (sb < total_sb) {
    uint8_t *blk = out + sb * 144u;
    *reinterpret_cast<uint4 *>(blk + 16u + 32u * (j >> 1) + 16u * (j & 1u)) =
        make_uint4(outw[0], outw[1], outw[2], outw[3]);
    if (j == 0u) *reinterpret_cast<uint4 *>(blk) = make_uint4(dh | (mh << 16), y, z, wq);
  }
}

}  // namespace

hipError_t launch_quantize_weight_q4k(const void *w_bf16, void *out, uint32_t n, uint32_t k,
                                      hipStream_t s) {
  const uint64_t total_sb = (uint64_t)n * (k >> 8);
  const uint64_t blocks = (total_sb * 8u + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(quantize_weight_q4k_kernel, dim3((uint32_t)blocks), dim3(kThreads), 0, s,
                     static_cast<const uint16_t *>(w_bf16), static_cast<uint8_t *>(out), total_sb);
  return hipGetLastError();
}

}  // namespace bqmm

// Q2_0 GEMV for decode (m = 1) and small verify batches (m = 2..8).
//
// [page layers/qwen3_ssm/init.rs, kernel q2_0_gemv_vec; page
//  layers/dense_ffn_decode_batch.rs, fn forward_km_q2: q2_0_gemv_vec_batchm on
//  the bf16 activations, output bf16.]
//
// out[i][r] = sum_k a[i][k] * d[r][g] * (c - 2), accumulated in fp32.
// A bandwidth kernel: the packed weight (2.125 bits per weight) is streamed
// once with 16-byte loads; no matrix cores.  16 lanes share one weight row;
// lane L owns the 16-byte half-groups L, L+16, ... of the row, i.e. 64 codes
// per load: for field j of byte t the code belongs to k = 128g + 32j + 16h + t.
#include "bqmm_internal.h"

namespace bqmm {
namespace {

constexpr int kLanesPerRow = 16;
constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / kLanesPerRow;

template <int M>
__global__ __launch_bounds__(kThreads) void q2_0_gemv_kernel(const uint16_t *__restrict__ act,
                                                             const uint8_t *__restrict__ w,
                                                             uint16_t *__restrict__ out,
                                                             uint32_t n, uint32_t k) {
  const uint32_t sub = threadIdx.x % kLanesPerRow;
  const uint32_t row = blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  const uint32_t chunks = k / 64u;  // 16-byte half-groups per row
  const uint16_t *scales = reinterpret_cast<const uint16_t *>(w + (uint64_t)n * k / 4u);

  float acc[M];
#pragma unroll
  for (int i = 0; i < M; ++i) acc[i] = 0.0f;

  if (row < n) {
    const uint8_t *wrow = w + (uint64_t)row * (k / 4u);
    for (uint32_t c = sub; c < chunks; c += kLanesPerRow) {
      const uint32_t g = c >> 1, h = c & 1u;
      const uint4 q = *reinterpret_cast<const uint4 *>(wrow + 16u * c);
      const float d = f16_bits_to_f32(scales[(uint64_t)row * (k / 128u) + g]);
      const uint32_t words[4] = {q.x, q.y, q.z, q.w};
      float part[M];
#pragma unroll
      for (int i = 0; i < M; ++i) part[i] = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t kbase = 128u * g + 32u * j + 16u * h;
#pragma unroll
        for (int i = 0; i < M; ++i) {
          const uint4 a0 = *reinterpret_cast<const uint4 *>(act + (uint64_t)i * k + kbase);
          const uint4 a1 = *reinterpret_cast<const uint4 *>(act + (uint64_t)i * k + kbase + 8);
          const uint32_t av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const uint32_t code = (words[t / 4] >> (8 * (t % 4) + 2 * j)) & 3u;
            const float wv = (float)((int)code - 2);
            const float av_f = (t & 1) ? __uint_as_float(av[t / 2] & 0xFFFF0000u)
                                       : __uint_as_float(av[t / 2] << 16);
            part[i] = fmaf(wv, av_f, part[i]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < M; ++i) acc[i] = fmaf(d, part[i], acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < M; ++i) {
#pragma unroll
    for (int off = kLanesPerRow / 2; off > 0; off >>= 1) acc[i] += __shfl_xor(acc[i], off);
  }
  if (row < n && sub == 0) {
#pragma unroll
    for (int i = 0; i < M; ++i) out[(uint64_t)i * n + row] = (uint16_t)f32_to_bf16_rne(acc[i]);
  }
}

template <int M>
hipError_t launch_m(const void *act, const void *w, void *out, uint32_t n, uint32_t k,
                    hipStream_t s) {
  const uint32_t blocks = (n + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(q2_0_gemv_kernel<M>, dim3(blocks), dim3(kThreads), 0, s,
                     static_cast<const uint16_t *>(act), static_cast<const uint8_t *>(w),
                     static_cast<uint16_t *>(out), n, k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_q2_0_gemv(const void *act, const void *w, void *out, uint32_t m, uint32_t n,
                            uint32_t k, hipStream_t s) {
  switch (m) {
    case 1: return launch_m<1>(act, w, out, n, k, s);
    case 2: return launch_m<2>(act, w, out, n, k, s);
    case 3: return launch_m<3>(act, w, out, n, k, s);
    case 4: return launch_m<4>(act, w, out, n, k, s);
    case 5: return launch_m<5>(act, w, out, n, k, s);
    case 6: return launch_m<6>(act, w, out, n, k, s);
    case 7: return launch_m<7>(act, w, out, n, k, s);
    case 8: return launch_m<8>(act, w, out, n, k, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bqmm

// Dense bf16 GEMM for the dequant fallback: out[m][n] = sum_k a[m][k] * w[n][k].
//
// [page layers/qwen3_ssm/init_q2.rs, fn qkvz_q2_prefill_gemm: when the MMQ
//  path is unavailable the weight is dequantized to BF16 scratch and
//  dense_gemm_bf16_pipelined runs on the original bf16 input.]
//
// bf16 matrix cores (v_mfma_f32_32x32x16_bf16), fp32 accumulation, bf16 out.
// Tile 128 (n) x 128 (m), 4 waves of 64 x 64, k staged 64 at a time through
// LDS.  The weight is the A operand so that a lane's 16 accumulators share
// one output row and are stored as four 8-byte runs.
#include "bqmm_internal.h"

namespace bqmm {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BN = 128, BM = 128, KS = 64;
constexpr int LDS_STRIDE = KS * 2 + 16;  // bytes per staged row
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void dense_gemm_bf16_kernel(
    const uint16_t *__restrict__ a, const uint16_t *__restrict__ w, uint16_t *__restrict__ out,
    uint32_t m, uint32_t n, uint32_t k) {
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint8_t w_lds[BN * LDS_STRIDE];
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint32_t wn = wave & 1u, wm = wave >> 1;
  const uint32_t n_base = blockIdx.x * BN, m_base = blockIdx.y * BM;

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  for (uint32_t k0 = 0; k0 < k; k0 += KS) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t c = tid + kThreads * i;
      const uint32_t r = c >> 3, col = (c & 7u) * 8u;  // 8 bf16 = 16 bytes
      uint4 va = make_uint4(0, 0, 0, 0), vw = make_uint4(0, 0, 0, 0);
      if (m_base + r < m) va = *reinterpret_cast<const uint4 *>(a + (uint64_t)(m_base + r) * k + k0 + col);
      if (n_base + r < n) vw = *reinterpret_cast<const uint4 *>(w + (uint64_t)(n_base + r) * k + k0 + col);
      *reinterpret_cast<uint4 *>(a_lds + r * LDS_STRIDE + col * 2) = va;
      *reinterpret_cast<uint4 *>(w_lds + r * LDS_STRIDE + col * 2) = vw;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KS / 16; ++kk) {
      v8bf A[2], B[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        A[s] = *reinterpret_cast<const v8bf *>(w_lds + (wn * 64 + s * 32 + (lane & 31)) * LDS_STRIDE + 32 * kk + 16 * (lane >> 5));
        B[s] = *reinterpret_cast<const v8bf *>(a_lds + (wm * 64 + s * 32 + (lane & 31)) * LDS_STRIDE + 32 * kk + 16 * (lane >> 5));
      }
#pragma unroll
      for (int sn = 0; sn < 2; ++sn)
#pragma unroll
        for (int sm = 0; sm < 2; ++sm)
          acc[sn][sm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[sn], B[sm], acc[sn][sm], 0, 0, 0);
    }
  }

  const bool vec = (n % 4u) == 0u;
#pragma unroll
  for (int sm = 0; sm < 2; ++sm) {
    const uint32_t mm = m_base + wm * 64 + sm * 32 + (lane & 31);
    if (mm >= m) continue;
    uint16_t *orow = out + (uint64_t)mm * n;
#pragma unroll
    for (int sn = 0; sn < 2; ++sn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t nn = n_base + wn * 64 + sn * 32 + 8 * q + 4 * (lane >> 5);
        const v16f &v = acc[sn][sm];
        if (vec && nn + 4 <= n) {
          *reinterpret_cast<uint2 *>(orow + nn) =
              make_uint2(pack_bf16x2(v[4 * q], v[4 * q + 1]), pack_bf16x2(v[4 * q + 2], v[4 * q + 3]));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (nn + e < n) orow[nn + e] = (uint16_t)f32_to_bf16_rne(v[4 * q + e]);
        }
      }
  }
}

}  // namespace

hipError_t launch_dense_gemm_bf16(const void *a, const void *w, void *out, uint32_t m, uint32_t n,
                                  uint32_t k, hipStream_t s) {
  const dim3 grid((n + BN - 1) / BN, (m + BM - 1) / BM);
  hipLaunchKernelGGL(dense_gemm_bf16_kernel, grid, dim3(kThreads), 0, s,
                     static_cast<const uint16_t *>(a), static_cast<const uint16_t *>(w),
                     static_cast<uint16_t *>(out), m, n, k);
  return hipGetLastError();
}

}  // namespace bqmm

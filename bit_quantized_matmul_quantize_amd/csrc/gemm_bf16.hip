// Dense bf16 GEMM for the dequant fallback: out[m][n] = sum_k a[m][k] * w[n][k].
//
// [page layers/qwen3_ssm/init_q2.rs, fn qkvz_q2_prefill_gemm: when the MMQ
//  path is unavailable the weight is dequantized to BF16 scratch and
//  dense_gemm_bf16_pipelined runs on the original bf16 input.]
//
// bf16 matrix cores (v_mfma_f32_32x32x16_bf16), fp32 accumulation, bf16 out.
// Tile 128 (n) x 128 (m), 4 waves of 64 x 64, k staged KS = 64 at a time
// through two LDS stages: while stage s is multiplied, the registers holding
// the global loads of step s + 1 are written into the other stage and the
// loads of step s + 2 are already in flight, so one barrier per step and no
// exposed load latency.  The weight is the A operand so that a lane's 16
// accumulators share one output row and are stored as four 8-byte runs.
// Rows past m or n load the last valid row and are not stored.
#include "bqmm_internal.h"

namespace bqmm {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BN = 128, BM = 128, KS = 64;
constexpr int LDS_STRIDE = KS * 2 + 16;  // bytes per staged row; the pad spreads banks
constexpr int kThreads = 256;
constexpr int kTileBytes = BM * LDS_STRIDE;      // one operand tile (128 rows)
constexpr int kStageBytes = 2 * kTileBytes;      // activation tile + weight tile
constexpr int kLoads = BM * KS * 2 / 16 / kThreads;  // 16-byte loads per thread per operand (4)

__global__ __launch_bounds__(kThreads, 2) void dense_gemm_bf16_kernel(
    const uint16_t *__restrict__ a, const uint16_t *__restrict__ w, uint16_t *__restrict__ out,
    uint32_t m, uint32_t n, uint32_t k) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint32_t wn = wave & 1u, wm = wave >> 1;
  // m tiles run consecutively (grid x), so the workgroups that share a weight
  // tile are co-resident and read it from L2 rather than from memory
  const uint32_t n_base = blockIdx.y * BN, m_base = blockIdx.x * BM;
  const uint32_t nsteps = k / KS;

  // This thread's rows and 16-byte column of each operand tile.  The staging
  // registers are named scalars: as arrays, indexed inside the macros' loops,
  // they were kept in scratch memory.
  static_assert(kLoads == 4, "four 16-byte loads per operand and thread");
  const uint32_t r0 = tid >> 3, col = (tid & 7u) * 8u;  // 8 bf16 = 16 bytes
  const uint16_t *ap = a + (uint64_t)min(m_base + r0, m - 1u) * k + col;
  const uint16_t *wp = w + (uint64_t)min(n_base + r0, n - 1u) * k + col;
  // rows r0 + 32 i; rows past m (n) read the last valid row
  const uint64_t ast[4] = {0, (uint64_t)(min(m_base + r0 + 32u, m - 1u) - min(m_base + r0, m - 1u)) * k,
                           (uint64_t)(min(m_base + r0 + 64u, m - 1u) - min(m_base + r0, m - 1u)) * k,
                           (uint64_t)(min(m_base + r0 + 96u, m - 1u) - min(m_base + r0, m - 1u)) * k};
  const uint64_t wst[4] = {0, (uint64_t)(min(n_base + r0 + 32u, n - 1u) - min(n_base + r0, n - 1u)) * k,
                           (uint64_t)(min(n_base + r0 + 64u, n - 1u) - min(n_base + r0, n - 1u)) * k,
                           (uint64_t)(min(n_base + r0 + 96u, n - 1u) - min(n_base + r0, n - 1u)) * k};
  const uint32_t soff = r0 * LDS_STRIDE + col * 2;
  constexpr uint32_t kRowStep = 32 * LDS_STRIDE;

  uint4 ra0, ra1, ra2, ra3, rw0, rw1, rw2, rw3;
#define BQMM_GLOAD(step)                                                              \
  do {                                                                                \
    const uint64_t o_ = (uint64_t)(step) * KS;                                        \
    ra0 = *reinterpret_cast<const uint4 *>(ap + ast[0] + o_);                         \
    ra1 = *reinterpret_cast<const uint4 *>(ap + ast[1] + o_);                         \
    ra2 = *reinterpret_cast<const uint4 *>(ap + ast[2] + o_);                         \
    ra3 = *reinterpret_cast<const uint4 *>(ap + ast[3] + o_);                         \
    rw0 = *reinterpret_cast<const uint4 *>(wp + wst[0] + o_);                         \
    rw1 = *reinterpret_cast<const uint4 *>(wp + wst[1] + o_);                         \
    rw2 = *reinterpret_cast<const uint4 *>(wp + wst[2] + o_);                         \
    rw3 = *reinterpret_cast<const uint4 *>(wp + wst[3] + o_);                         \
  } while (0)
#define BQMM_STORE(st)                                                                \
  do {                                                                                \
    uint8_t *a_l = lds + (st) * kStageBytes + soff, *w_l = a_l + kTileBytes;          \
    *reinterpret_cast<uint4 *>(a_l) = ra0;                                            \
    *reinterpret_cast<uint4 *>(a_l + kRowStep) = ra1;                                 \
    *reinterpret_cast<uint4 *>(a_l + 2 * kRowStep) = ra2;                             \
    *reinterpret_cast<uint4 *>(a_l + 3 * kRowStep) = ra3;                             \
    *reinterpret_cast<uint4 *>(w_l) = rw0;                                            \
    *reinterpret_cast<uint4 *>(w_l + kRowStep) = rw1;                                 \
    *reinterpret_cast<uint4 *>(w_l + 2 * kRowStep) = rw2;                             \
    *reinterpret_cast<uint4 *>(w_l + 3 * kRowStep) = rw3;                             \
  } while (0)

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  BQMM_GLOAD(0u);
  BQMM_STORE(0);
  if (nsteps > 1) BQMM_GLOAD(1u);
  for (uint32_t s = 0; s < nsteps; ++s) {
    __syncthreads();  // stage s is complete; nobody still reads stage s + 1's buffer
    if (s + 1 < nsteps) {
      BQMM_STORE((s + 1) & 1u);
      if (s + 2 < nsteps) BQMM_GLOAD(s + 2);
    }
    const uint8_t *a_l = lds + (s & 1u) * kStageBytes, *w_l = a_l + kTileBytes;
#pragma unroll
    for (int kk = 0; kk < KS / 16; ++kk) {
      v8bf A[2], B[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        A[t] = *reinterpret_cast<const v8bf *>(w_l + (wn * 64 + t * 32 + (lane & 31)) * LDS_STRIDE + 32 * kk + 16 * (lane >> 5));
        B[t] = *reinterpret_cast<const v8bf *>(a_l + (wm * 64 + t * 32 + (lane & 31)) * LDS_STRIDE + 32 * kk + 16 * (lane >> 5));
      }
#pragma unroll
      for (int sn = 0; sn < 2; ++sn)
#pragma unroll
        for (int sm = 0; sm < 2; ++sm)
          acc[sn][sm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[sn], B[sm], acc[sn][sm], 0, 0, 0);
    }
  }
#undef BQMM_GLOAD
#undef BQMM_STORE

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
  // two stages (73.7 KB) exceed the 64 KB default dynamic-LDS limit
  const hipError_t attr_err = ensure_dynamic_lds(reinterpret_cast<const void *>(dense_gemm_bf16_kernel),
                                                 2 * kStageBytes);
  if (attr_err != hipSuccess) return attr_err;
  const dim3 grid((m + BM - 1) / BM, (n + BN - 1) / BN);
  hipLaunchKernelGGL(dense_gemm_bf16_kernel, grid, dim3(kThreads), 2 * kStageBytes, s,
                     static_cast<const uint16_t *>(a), static_cast<const uint16_t *>(w),
                     static_cast<uint16_t *>(out), m, n, k);
  return hipGetLastError();
}

}  // namespace bqmm

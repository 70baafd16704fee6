// Dense bf16 GEMM for the dequant fallback: out[m][n] = sum_k a[m][k] * w[n][k].
//
// [page layers/qwen3_ssm/init_q2.rs, fn qkvz_q2_prefill_gemm: when the MMQ
//  path is unavailable the weight is dequantized to BF16 scratch and
//  dense_gemm_bf16_pipelined runs on the original bf16 input.]
//
// bf16 matrix cores (v_mfma_f32_32x32x16_bf16), fp32 accumulation, bf16 out.
// Tile BN (n) x 128 (m): 128 x 128 with 4 waves of 64 x 64, or 96 x 128 with
// 4 waves of 96 x 32 where that fills the chip in fewer rounds of
// workgroups (the same choice as the MMQ's).  k is staged KS = 64 at a time
// through two LDS stages: after stage s's operands are read, the registers
// holding the global loads of step s + 1 are written into the other stage and
// the loads of step s + 2 are issued, so one barrier per step and no exposed
// load latency.  The weight is the A operand so that a lane's 16
// accumulators share one output row and are stored as four 8-byte runs.
// Rows past m or n load the last valid row and are not stored.
#include "bqmm_internal.h"

namespace bqmm {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BM = 128, KS = 64;
constexpr int LDS_STRIDE = KS * 2 + 16;  // bytes per staged row; the pad spreads banks
constexpr int kThreads = 256;
constexpr int kTileBytes = BM * LDS_STRIDE;      // the activation tile (128 rows)
constexpr int kLoads = BM * KS * 2 / 16 / kThreads;  // 16-byte loads per thread per 128 rows (4)
// one LDS stage: activation tile + weight tile of bn rows
__host__ __device__ constexpr int stage_bytes(int bn) { return kTileBytes + bn * LDS_STRIDE; }

// TN x TM subtiles of 32 x 32 per wave, WN waves along n (4 / WN along m).
template <int TN, int TM, int WN>
__global__ __launch_bounds__(kThreads, 2) void dense_gemm_bf16_kernel(
    const uint16_t *__restrict__ a, const uint16_t *__restrict__ w, uint16_t *__restrict__ out,
    uint32_t m, uint32_t n, uint32_t k) {
  constexpr int WM = 4 / WN;
  constexpr int BN = 32 * TN * WN;
  static_assert(WN * WM == 4 && 32 * TM * WM == BM, "four waves cover 128 activation rows");
  static_assert(BN == 128 || BN == 96, "three or four 32-row weight loads per thread");
  constexpr int kStageBytes = stage_bytes(BN);
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint32_t wn = wave % WN, wm = wave / WN;
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
    if constexpr (BN == 128) rw3 = *reinterpret_cast<const uint4 *>(wp + wst[3] + o_); \
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
    if constexpr (BN == 128) *reinterpret_cast<uint4 *>(w_l + 3 * kRowStep) = rw3;    \
  } while (0)

  v16f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  BQMM_GLOAD(0u);
  BQMM_STORE(0);
  if (nsteps > 1) BQMM_GLOAD(1u);
  for (uint32_t s = 0; s < nsteps; ++s) {
    __syncthreads();  // stage s is complete; nobody still reads stage s + 1's buffer
    const uint8_t *a_l = lds + (s & 1u) * kStageBytes, *w_l = a_l + kTileBytes;
    // Per step: every operand of the step is read from LDS first, then the
    // next stage is written from registers (its LDS writes queue behind the
    // reads, so the first MFMA does not wait for them; 11-13% faster than
    // writing first), then the MFMAs run.
    v8bf A[KS / 16][TN], B[KS / 16][TM];
#pragma unroll
    for (int kk = 0; kk < KS / 16; ++kk) {
#pragma unroll
      for (int t = 0; t < TN; ++t)
        A[kk][t] = *reinterpret_cast<const v8bf *>(w_l + (wn * (32 * TN) + t * 32 + (lane & 31)) * LDS_STRIDE + 32 * kk + 16 * (lane >> 5));
#pragma unroll
      for (int t = 0; t < TM; ++t)
        B[kk][t] = *reinterpret_cast<const v8bf *>(a_l + (wm * (32 * TM) + t * 32 + (lane & 31)) * LDS_STRIDE + 32 * kk + 16 * (lane >> 5));
    }
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < nsteps) {
      BQMM_STORE((s + 1) & 1u);
      if (s + 2 < nsteps) BQMM_GLOAD(s + 2);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < KS / 16; ++kk)
#pragma unroll
      for (int sn = 0; sn < TN; ++sn)
#pragma unroll
        for (int sm = 0; sm < TM; ++sm)
          acc[sn][sm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[kk][sn], B[kk][sm], acc[sn][sm], 0, 0, 0);
  }
#undef BQMM_GLOAD
#undef BQMM_STORE

  const bool vec = (n % 4u) == 0u;
#pragma unroll
  for (int sm = 0; sm < TM; ++sm) {
    const uint32_t mm = m_base + wm * (32 * TM) + sm * 32 + (lane & 31);
    if (mm >= m) continue;
    uint16_t *orow = out + (uint64_t)mm * n;
#pragma unroll
    for (int sn = 0; sn < TN; ++sn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t nn = n_base + wn * (32 * TN) + sn * 32 + 8 * q + 4 * (lane >> 5);
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

template <int TN, int TM, int WN>
hipError_t launch_dense_layout(const void *a, const void *w, void *out, uint32_t m, uint32_t n, uint32_t k,
                               hipStream_t s) {
  constexpr int BN = 32 * TN * WN;
  constexpr int lds = 2 * stage_bytes(BN);
  // two stages (64.5 KB, 73.7 KB) exceed the 64 KB default dynamic-LDS limit
  const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void *>(dense_gemm_bf16_kernel<TN, TM, WN>), lds);
  if (e != hipSuccess) return e;
  const dim3 grid((uint32_t)(((uint64_t)m + BM - 1) / BM), (uint32_t)(((uint64_t)n + BN - 1) / BN));
  hipLaunchKernelGGL((dense_gemm_bf16_kernel<TN, TM, WN>), grid, dim3(kThreads), lds, s,
                     static_cast<const uint16_t *>(a), static_cast<const uint16_t *>(w),
                     static_cast<uint16_t *>(out), m, n, k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_gemm_bf16(const void *a, const void *w, void *out, uint32_t m, uint32_t n,
                                  uint32_t k, hipStream_t s) {
  int cus = 0;
  const hipError_t e = device_cu_count(&cus);
  if (e != hipSuccess) return e;
  // Rounds of resident workgroups (two per CU); 96 x 128 tiles hold 3/4 of
  // the work of 128 x 128 tiles.
  const uint64_t slots = 2ull * (uint64_t)(cus > 0 ? cus : 1);
  const uint64_t tiles_m = ((uint64_t)m + BM - 1) / BM;
  const uint64_t tiles96 = (n + 95ull) / 96ull;
  const uint64_t rounds128 = ((n + 127ull) / 128ull * tiles_m + slots - 1) / slots;
  const uint64_t rounds96 = (tiles96 * tiles_m + slots - 1) / slots;
  // (n tiles are the second grid dimension, at most 65535)
  if (3 * rounds96 < 4 * rounds128 && tiles96 <= 65535u) return launch_dense_layout<3, 1, 1>(a, w, out, m, n, k, s);
  return launch_dense_layout<2, 2, 2>(a, w, out, m, n, k, s);
}

}  // namespace bqmm

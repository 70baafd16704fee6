// Q4_K x q8_1 MMQ on CDNA4 matrix cores.
//
// [page layers/ops/q4k_mmq.rs, fn q4k_mmq_gemm: C[m, n] = A[m, k] x W[n, k]
//  with A in q8_1 and W in block_q4_K (256 weights in 144 bytes), BF16 store,
//  any n (a with-check variant for n % 128 != 0).]
//
// out[m][n] = sum_j da[m][j] * d[n]*sc_j[n] * D[m][n][j]  -  sum_j dmin[n]*m_j[n] * s[m][j]
//   D = sum_{t<32} q4 * q (exact int32, one 32-block),  s = the stored q8_1 sum (da * sum q).
//
// Tile 128 (n) x 256 (m), 512 lanes = 8 waves of 64 (n) x 64 (m); k is staged
// 128 at a time (half a super-block: four sub-blocks) through two LDS stages.
//   * main term: v_mfma_i32_32x32x32_i8 per sub-block (weights as A, so a
//     lane's 16 accumulators share one activation row and da is a lane
//     value), then per output: float(D) * da, times d*sc_j of its weight row
//     (from LDS), added into the output accumulator;
//   * min term: one v_mfma_f32_32x32x8_f16 per stage and subtile with
//     A = fp16(-dmin * m_j) for the stage's four sub-blocks and B = their s,
//     accumulating into the same output registers (no VALU).
// The MFMA of step i + 1 is issued before the epilogue of step i, and the
// compute is last in the loop body (see the Q2_0 kernel for why).
#include "bqmm_internal.h"

namespace bqmm {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

constexpr int BN = 128;
constexpr int BM = 256;
constexpr int KG = 128;
constexpr int LDS_STRIDE = KG + 16;
constexpr int kThreads = 512;
// one LDS stage
constexpr int kActBytes = BM * LDS_STRIDE;          // activation codes
constexpr int kWBytes = BN * LDS_STRIDE;            // weight codes (one byte each)
constexpr int kDscOff = kActBytes + kWBytes;        // float [4][BN]: d * sc_j
constexpr int kNminOff = kDscOff + 4 * BN * 4;      // fp16 [BN][4]: -dmin * m_j
constexpr int kDaOff = kNminOff + BN * 8;           // float [BM][4]: da
constexpr int kSOff = kDaOff + BM * 16;             // fp16 [BM][4]: s
constexpr int kStageBytes = kSOff + BM * 8;

__device__ __forceinline__ void scale_min(const uint32_t S[3], int j, uint32_t &sc, uint32_t &mn) {
  auto byte = [&](int i) { return (S[i >> 2] >> (8 * (i & 3))) & 0xFFu; };
  if (j < 4) {
    sc = byte(j) & 63u;
    mn = byte(j + 4) & 63u;
  } else {
    sc = (byte(j + 4) & 15u) | ((byte(j - 4) >> 6) << 4);
    mn = (byte(j + 4) >> 4) | ((byte(j) >> 6) << 4);
  }
}

template <bool kDump>
__global__ __launch_bounds__(kThreads, 1) void q4k_mmq_kernel(
    const uint8_t *__restrict__ act_q8, const uint8_t *__restrict__ w, uint16_t *__restrict__ out,
    int32_t *__restrict__ dots, uint32_t m, uint32_t n, uint32_t k, uint32_t m0, uint32_t mt,
    uint32_t n0, uint32_t nt, uint32_t tile_n0, uint32_t tile_m0, uint32_t ldc) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u, l32 = lane & 31u, hi = lane >> 5;
  const uint32_t wave = tid >> 6;
  const uint32_t wn = wave & 1u, wm = wave >> 1;  // wm in 0..3
  const uint32_t n_base = (blockIdx.x + tile_n0) * BN;
  const uint32_t m_base = (blockIdx.y + tile_m0) * BM;
  const uint32_t kpad = (k + 255u) / 256u * 256u;
  const uint32_t nblk_pad = kpad / 32u;
  const uint32_t nsb = k / 256u;
  const uint32_t nstages = k / KG;
  const uint8_t *ds = act_q8 + (uint64_t)m * kpad;

  // global -> register staging; rows past m or n read the last valid row
  uint32_t a_row[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a_row[i] = min(m_base + 64u * i + (tid >> 3), m - 1u);
  const uint32_t a_col = (tid & 7u) * 16u;
  const uint32_t w_row = min(n_base + (tid >> 2), n - 1u), w_part = tid & 3u;
  const uint32_t h_row = min(n_base + tid, n - 1u);         // header row for tid < BN
  const uint32_t s_row = min(m_base + (tid - 256u), m - 1u);  // activation-scale row for tid >= 256

  uint4 ra0, ra1, ra2, ra3, rw, rh = make_uint4(0, 0, 0, 0), rds = make_uint4(0, 0, 0, 0);
#define BQMM_FETCH(st)                                                                                  \
  do {                                                                                                  \
    const uint32_t sb_ = (st) >> 1, hs_ = (st) & 1u;                                                    \
    ra0 = *reinterpret_cast<const uint4 *>(act_q8 + (uint64_t)a_row[0] * kpad + (st) * KG + a_col);      \
    ra1 = *reinterpret_cast<const uint4 *>(act_q8 + (uint64_t)a_row[1] * kpad + (st) * KG + a_col);      \
    ra2 = *reinterpret_cast<const uint4 *>(act_q8 + (uint64_t)a_row[2] * kpad + (st) * KG + a_col);      \
    ra3 = *reinterpret_cast<const uint4 *>(act_q8 + (uint64_t)a_row[3] * kpad + (st) * KG + a_col);      \
    rw = *reinterpret_cast<const uint4 *>(w + ((uint64_t)w_row * nsb + sb_) * 144u + 16u + 64u * hs_ +  \
                                          16u * w_part);                                                \
    if (tid < BN)                                                                                       \
      rh = *reinterpret_cast<const uint4 *>(w + ((uint64_t)h_row * nsb + sb_) * 144u);                  \
    else if (tid >= 256u)                                                                               \
      rds = *reinterpret_cast<const uint4 *>(ds + 4ull * ((uint64_t)s_row * nblk_pad + 4u * (st)));     \
  } while (0)

#define BQMM_STAGE(buf, st)                                                                             \
  do {                                                                                                  \
    uint8_t *L = lds + (buf) * kStageBytes;                                                             \
    *reinterpret_cast<uint4 *>(L + (0 * 64 + (tid >> 3)) * LDS_STRIDE + a_col) = ra0;                   \
    *reinterpret_cast<uint4 *>(L + (1 * 64 + (tid >> 3)) * LDS_STRIDE + a_col) = ra1;                   \
    *reinterpret_cast<uint4 *>(L + (2 * 64 + (tid >> 3)) * LDS_STRIDE + a_col) = ra2;                   \
    *reinterpret_cast<uint4 *>(L + (3 * 64 + (tid >> 3)) * LDS_STRIDE + a_col) = ra3;                   \
    {                                                                                                   \
      /* part p: chunk tt = p / 2 (sub-blocks 2tt low nibbles, 2tt+1 high), bytes 16*(p%2) */          \
      const uint32_t tt = w_part >> 1, i0 = (w_part & 1u) * 16u;                                        \
      uint8_t *wr = L + kActBytes + (tid >> 2) * LDS_STRIDE + 64u * tt + i0;                            \
      *reinterpret_cast<uint4 *>(wr) = make_uint4(rw.x & 0x0F0F0F0Fu, rw.y & 0x0F0F0F0Fu,               \
                                                  rw.z & 0x0F0F0F0Fu, rw.w & 0x0F0F0F0Fu);              \
      *reinterpret_cast<uint4 *>(wr + 32) = make_uint4((rw.x >> 4) & 0x0F0F0F0Fu, (rw.y >> 4) & 0x0F0F0F0Fu, \
                                                       (rw.z >> 4) & 0x0F0F0F0Fu, (rw.w >> 4) & 0x0F0F0F0Fu); \
    }                                                                                                   \
    if (tid < BN) {                                                                                     \
      const float d_ = f16_bits_to_f32(rh.x & 0xFFFFu), dmin_ = f16_bits_to_f32(rh.x >> 16);           \
      const uint32_t S_[3] = {rh.y, rh.z, rh.w};                                                        \
      float *dsc = reinterpret_cast<float *>(L + kDscOff);                                              \
      _Float16 nm[4];                                                                                   \
      _Pragma("unroll") for (int jl = 0; jl < 4; ++jl) {                                                \
        uint32_t sc_, mn_;                                                                              \
        scale_min(S_, 4 * (int)((st) & 1u) + jl, sc_, mn_);                                             \
        dsc[jl * BN + tid] = d_ * (float)sc_;                                                           \
        nm[jl] = (_Float16)(-dmin_ * (float)mn_);                                                       \
      }                                                                                                 \
      *reinterpret_cast<v4h *>(L + kNminOff + tid * 8) = v4h{nm[0], nm[1], nm[2], nm[3]};               \
    } else if (tid >= 256u) {                                                                           \
      const uint32_t r_ = tid - 256u;                                                                   \
      *reinterpret_cast<float4 *>(L + kDaOff + r_ * 16) =                                               \
          make_float4(f16_bits_to_f32(rds.x & 0xFFFFu), f16_bits_to_f32(rds.y & 0xFFFFu),               \
                      f16_bits_to_f32(rds.z & 0xFFFFu), f16_bits_to_f32(rds.w & 0xFFFFu));              \
      *reinterpret_cast<uint2 *>(L + kSOff + r_ * 8) =                                                  \
          make_uint2((rds.x >> 16) | (rds.y & 0xFFFF0000u), (rds.z >> 16) | (rds.w & 0xFFFF0000u));     \
    }                                                                                                   \
  } while (0)

  v16f acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;
  const v16i zero16 = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

  BQMM_FETCH(0u);
  BQMM_STAGE(0u, 0u);
  if (nstages > 1) BQMM_FETCH(1u);
  for (uint32_t st = 0; st < nstages; ++st) {
    __syncthreads();
    if (st + 1 < nstages) {
      BQMM_STAGE((st + 1) & 1u, st + 1);
      if (st + 2 < nstages) BQMM_FETCH(st + 2);
    }
    const uint8_t *L = lds + (st & 1u) * kStageBytes;
    const uint8_t *a_lds = L, *w_lds = L + kActBytes;
    const float *dsc_lds = reinterpret_cast<const float *>(L + kDscOff);

    v4i A[2][4], B[2][4];
    float da[2][4];
#pragma unroll
    for (int sm = 0; sm < 2; ++sm) {
      const uint32_t ml = wm * 64 + sm * 32 + l32;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        B[sm][b] = *reinterpret_cast<const v4i *>(a_lds + ml * LDS_STRIDE + 32 * b + 16 * hi);
      const float4 t = *reinterpret_cast<const float4 *>(L + kDaOff + ml * 16);
      da[sm][0] = t.x; da[sm][1] = t.y; da[sm][2] = t.z; da[sm][3] = t.w;
    }
#pragma unroll
    for (int sn = 0; sn < 2; ++sn) {
      const uint32_t nl = wn * 64 + sn * 32 + l32;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        A[sn][b] = *reinterpret_cast<const v4i *>(w_lds + nl * LDS_STRIDE + 32 * b + 16 * hi);
    }
    if constexpr (!kDump) {
      // min term on the matrix core: K = 8 with the upper four k-slots zero
#pragma unroll
      for (int sn = 0; sn < 2; ++sn) {
        const uint32_t nl = wn * 64 + sn * 32 + l32;
        const v4h zh = {0, 0, 0, 0};
        const v4h an = hi ? zh : *reinterpret_cast<const v4h *>(L + kNminOff + nl * 8);
#pragma unroll
        for (int sm = 0; sm < 2; ++sm) {
          const uint32_t ml = wm * 64 + sm * 32 + l32;
          const v4h bs = hi ? zh : *reinterpret_cast<const v4h *>(L + kSOff + ml * 8);
          acc[sn][sm] = __builtin_amdgcn_mfma_f32_32x32x8f16(an, bs, acc[sn][sm], 0, 0, 0);
        }
      }
    }

    // 16 steps (sn, sm, b), software-pipelined by one
    v16i D[2];
    float dsc[16];
#pragma unroll
    for (int i = 0; i <= 16; ++i) {
      if (i < 16) {
        const int sn = i >> 3, sm = (i >> 2) & 1, b = i & 3;
        D[i & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[sn][b], B[sm][b], zero16, 0, 0, 0);
        // keep the MFMA ahead of the previous step's epilogue (see mmq_q2.hip)
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i > 0) {
        const int p = i - 1;
        const int sn = p >> 3, sm = (p >> 2) & 1, b = p & 3;
        const v16i &Dp = D[p & 1];
        if constexpr (kDump) {
          const uint32_t mm = m_base + wm * 64 + sm * 32 + l32;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t nn = n_base + wn * 64 + sn * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (mm >= m0 && mm < m0 + mt && nn >= n0 && nn < n0 + nt)
              dots[((uint64_t)(mm - m0) * nt + (nn - n0)) * (k / 32u) + 4u * st + b] = Dp[r];
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 t = *reinterpret_cast<const float4 *>(dsc_lds + b * BN + wn * 64 + sn * 32 + 8 * q + 4 * hi);
            dsc[4 * q + 0] = t.x; dsc[4 * q + 1] = t.y; dsc[4 * q + 2] = t.z; dsc[4 * q + 3] = t.w;
          }
          const float a = da[sm][b];
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[sn][sm][r] = fmaf((float)Dp[r] * a, dsc[r], acc[sn][sm][r]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#undef BQMM_FETCH
#undef BQMM_STAGE

  if constexpr (!kDump) {
    const bool full = (m_base + BM <= m) && (n_base + BN <= n) && (ldc % 4u) == 0u;
#pragma unroll
    for (int sm = 0; sm < 2; ++sm) {
      const uint32_t mm = m_base + wm * 64 + sm * 32 + l32;
      uint16_t *orow = out + (uint64_t)min(mm, m - 1u) * ldc;
#pragma unroll
      for (int sn = 0; sn < 2; ++sn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t nn = n_base + wn * 64 + sn * 32 + 8 * q + 4 * hi;
          const v16f &v = acc[sn][sm];
          if (full) {
            *reinterpret_cast<uint2 *>(orow + nn) =
                make_uint2(pack_bf16x2(v[4 * q], v[4 * q + 1]), pack_bf16x2(v[4 * q + 2], v[4 * q + 3]));
          } else if (mm < m) {
            if ((ldc % 4u) == 0u && nn + 4 <= n) {
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
  }
}

}  // namespace

hipError_t launch_q4k_mmq(const void *act_q8, const void *w, void *out, int32_t *dots,
                          uint32_t m0, uint32_t mt, uint32_t n0, uint32_t nt, uint32_t m,
                          uint32_t n, uint32_t k, uint32_t ldc, hipStream_t s) {
  // Two stages exceed the 64 KB default dynamic-LDS limit; gfx950 allows 160 KB.
  hipError_t attr_err = ensure_dynamic_lds(reinterpret_cast<const void *>(q4k_mmq_kernel<false>), 2 * kStageBytes);
  if (attr_err == hipSuccess)
    attr_err = ensure_dynamic_lds(reinterpret_cast<const void *>(q4k_mmq_kernel<true>), 2 * kStageBytes);
  if (attr_err != hipSuccess) return attr_err;
  if (dots == nullptr) {
    const dim3 grid((uint32_t)(((uint64_t)n + BN - 1) / BN), (uint32_t)(((uint64_t)m + BM - 1) / BM));
    hipLaunchKernelGGL(q4k_mmq_kernel<false>, grid, dim3(kThreads), 2 * kStageBytes, s,
                       static_cast<const uint8_t *>(act_q8), static_cast<const uint8_t *>(w),
                       static_cast<uint16_t *>(out), nullptr, m, n, k, 0u, 0u, 0u, 0u, 0u, 0u, ldc);
  } else {
    const uint32_t tn0 = n0 / BN, tn1 = (n0 + nt - 1) / BN;
    const uint32_t tm0 = m0 / BM, tm1 = (m0 + mt - 1) / BM;
    const dim3 grid(tn1 - tn0 + 1, tm1 - tm0 + 1);
    hipLaunchKernelGGL(q4k_mmq_kernel<true>, grid, dim3(kThreads), 2 * kStageBytes, s,
                       static_cast<const uint8_t *>(act_q8), static_cast<const uint8_t *>(w),
                       nullptr, dots, m, n, k, m0, mt, n0, nt, tn0, tm0, n);
  }
  return hipGetLastError();
}

}  // namespace bqmm

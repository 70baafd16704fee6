// Q4_K x q8_1 MMQ on CDNA4 int8 matrix cores.
//
// [page layers/ops/q4k_mmq.rs, fn q4k_mmq_gemm: C[m, n] = A[m, k] x W[n, k]
//  with A in q8_1 and W in block_q4_K (256 weights in 144 bytes), BF16 store,
//  any n (a with-check variant for n % 128 != 0).]
//
// out[m][n] = sum_j da[m][j] * ( d*sc_j[n] * D[m][n][j] - dmin*m_j[n] * Q[m][j] ),
//   D = sum_{t<32} q4 * q (exact int32),  da * Q is the stored q8_1 sum s.
//
// Same tiling as the Q2_0 kernel: 128 x 128 tile, 4 waves of 64 x 64,
// v_mfma_i32_32x32x32_i8 with the weights as A so that a lane's accumulators
// share one activation row.  A stage is half a super-block (128 k = four
// sub-blocks): its 64 code bytes per weight row are split into low and high
// nibbles in LDS, and the four sub-blocks' d*sc and dmin*m go to LDS as fp32.
#include "bqmm_internal.h"

namespace bqmm {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BN = 128;
constexpr int BM = 128;
constexpr int KG = 128;
constexpr int LDS_STRIDE = KG + 16;
constexpr int kThreads = 256;

template <bool kDump>
__global__ __launch_bounds__(kThreads) void q4k_mmq_kernel(
    const uint8_t *__restrict__ act_q8, const uint8_t *__restrict__ w, uint16_t *__restrict__ out,
    int32_t *__restrict__ dots, uint32_t m, uint32_t n, uint32_t k, uint32_t m0, uint32_t mt,
    uint32_t n0, uint32_t nt, uint32_t tile_n0, uint32_t tile_m0) {
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint8_t w_lds[BN * LDS_STRIDE];
  __shared__ float dsc_lds[4][BN];
  __shared__ float dmn_lds[4][BN];
  __shared__ float da_lds[BM * 4];
  __shared__ float sa_lds[BM * 4];

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = tid >> 6;
  const uint32_t wn = wave & 1u, wm = wave >> 1;
  const uint32_t n_base = (blockIdx.x + tile_n0) * BN;
  const uint32_t m_base = (blockIdx.y + tile_m0) * BM;
  const uint32_t kpad = (k + 255u) / 256u * 256u;
  const uint32_t nblk_pad = kpad / 32u;
  const uint32_t nsb = k / 256u;
  const uint32_t nstages = k / KG;
  const uint8_t *ds = act_q8 + (uint64_t)m * kpad;

  float acc[2][2][16], accm[2][2][16];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = accm[a][b][r] = 0.0f;

  const v16i zero16 = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

  for (uint32_t st = 0; st < nstages; ++st) {
    const uint32_t sb = st >> 1, hs = st & 1u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t c = tid + kThreads * i;
      const uint32_t r = c >> 3, col = (c & 7u) * 16u;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m_base + r < m)
        v = *reinterpret_cast<const uint4 *>(act_q8 + (uint64_t)(m_base + r) * kpad + st * KG + col);
      *reinterpret_cast<uint4 *>(a_lds + r * LDS_STRIDE + col) = v;
    }
    {
      // codes: chunk tt (0/1) of this half holds sub-blocks 2tt (low nibbles) and 2tt+1 (high)
      const uint32_t r = tid >> 1, tt = tid & 1u;
      const uint8_t *blk = w + ((uint64_t)(n_base + r) * nsb + sb) * 144u;
#pragma unroll
      for (int i0 = 0; i0 < 32; i0 += 16) {
        uint4 p = make_uint4(0, 0, 0, 0);
        if (n_base + r < n) p = *reinterpret_cast<const uint4 *>(blk + 16u + 64u * hs + 32u * tt + i0);
        const uint4 lo = make_uint4(p.x & 0x0F0F0F0Fu, p.y & 0x0F0F0F0Fu, p.z & 0x0F0F0F0Fu, p.w & 0x0F0F0F0Fu);
        const uint4 hi = make_uint4((p.x >> 4) & 0x0F0F0F0Fu, (p.y >> 4) & 0x0F0F0F0Fu,
                                    (p.z >> 4) & 0x0F0F0F0Fu, (p.w >> 4) & 0x0F0F0F0Fu);
        *reinterpret_cast<uint4 *>(w_lds + r * LDS_STRIDE + 64 * tt + i0) = lo;
        *reinterpret_cast<uint4 *>(w_lds + r * LDS_STRIDE + 64 * tt + 32 + i0) = hi;
      }
    }
    if (tid < BN) {
      const uint32_t r = tid;
      float dsc[4] = {0, 0, 0, 0}, dmn[4] = {0, 0, 0, 0};
      if (n_base + r < n) {
        const uint4 h = *reinterpret_cast<const uint4 *>(w + ((uint64_t)(n_base + r) * nsb + sb) * 144u);
        const float d = f16_bits_to_f32(h.x & 0xFFFFu);
        const float dmin = f16_bits_to_f32(h.x >> 16);
        uint8_t S[12];
        const uint32_t sw[3] = {h.y, h.z, h.w};
#pragma unroll
        for (int i = 0; i < 12; ++i) S[i] = (uint8_t)(sw[i / 4] >> (8 * (i % 4)));
#pragma unroll
        for (int jl = 0; jl < 4; ++jl) {
          const int j = 4 * (int)hs + jl;
          uint32_t sc, mn;
          if (j < 4) {
            sc = S[j] & 63u;
            mn = S[j + 4] & 63u;
          } else {
            sc = (uint32_t)(S[j + 4] & 15u) | ((uint32_t)(S[j - 4] >> 6) << 4);
            mn = (uint32_t)(S[j + 4] >> 4) | ((uint32_t)(S[j] >> 6) << 4);
          }
          dsc[jl] = d * (float)sc;
          dmn[jl] = dmin * (float)mn;
        }
      }
#pragma unroll
      for (int jl = 0; jl < 4; ++jl) {
        dsc_lds[jl][r] = dsc[jl];
        dmn_lds[jl][r] = dmn[jl];
      }
    } else {
      const uint32_t r = tid - BN;
      float da[4] = {0, 0, 0, 0}, sa[4] = {0, 0, 0, 0};
      if (m_base + r < m) {
        const uint4 pr = *reinterpret_cast<const uint4 *>(ds + 4ull * ((uint64_t)(m_base + r) * nblk_pad + 4u * st));
        const uint32_t pv[4] = {pr.x, pr.y, pr.z, pr.w};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          da[b] = f16_bits_to_f32(pv[b] & 0xFFFFu);
          sa[b] = f16_bits_to_f32(pv[b] >> 16);
        }
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        da_lds[r * 4 + b] = da[b];
        sa_lds[r * 4 + b] = sa[b];
      }
    }
    __syncthreads();

#pragma unroll
    for (int b = 0; b < 4; ++b) {
      v4i A[2], B[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        A[s] = *reinterpret_cast<const v4i *>(w_lds + (wn * 64 + s * 32 + (lane & 31)) * LDS_STRIDE + 32 * b + 16 * (lane >> 5));
        B[s] = *reinterpret_cast<const v4i *>(a_lds + (wm * 64 + s * 32 + (lane & 31)) * LDS_STRIDE + 32 * b + 16 * (lane >> 5));
      }
      float dsc[2][16], dmn[2][16];
      if constexpr (!kDump) {
#pragma unroll
        for (int sn = 0; sn < 2; ++sn)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t nl = wn * 64 + sn * 32 + 8 * q + 4 * (lane >> 5);
            const float4 t = *reinterpret_cast<const float4 *>(&dsc_lds[b][nl]);
            const float4 u = *reinterpret_cast<const float4 *>(&dmn_lds[b][nl]);
            dsc[sn][4 * q] = t.x; dsc[sn][4 * q + 1] = t.y; dsc[sn][4 * q + 2] = t.z; dsc[sn][4 * q + 3] = t.w;
            dmn[sn][4 * q] = u.x; dmn[sn][4 * q + 1] = u.y; dmn[sn][4 * q + 2] = u.z; dmn[sn][4 * q + 3] = u.w;
          }
      }
#pragma unroll
      for (int sn = 0; sn < 2; ++sn)
#pragma unroll
        for (int sm = 0; sm < 2; ++sm) {
          const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[sn], B[sm], zero16, 0, 0, 0);
          const uint32_t ml = wm * 64 + sm * 32 + (lane & 31);
          if constexpr (kDump) {
            const uint32_t mm = m_base + ml;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const uint32_t nn = n_base + wn * 64 + sn * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
              if (mm >= m0 && mm < m0 + mt && nn >= n0 && nn < n0 + nt)
                dots[((uint64_t)(mm - m0) * nt + (nn - n0)) * (k / 32u) + 4u * st + b] = D[r];
            }
          } else {
            const float da = da_lds[ml * 4 + b];
            const float sa = sa_lds[ml * 4 + b];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              acc[sn][sm][r] = fmaf((float)D[r] * da, dsc[sn][r], acc[sn][sm][r]);
              accm[sn][sm][r] = fmaf(dmn[sn][r], sa, accm[sn][sm][r]);
            }
          }
        }
    }
  }

  if constexpr (!kDump) {
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
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[sn][sm][4 * q + e] - accm[sn][sm][4 * q + e];
          if (vec && nn + 4 <= n) {
            *reinterpret_cast<uint2 *>(orow + nn) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (nn + e < n) orow[nn + e] = (uint16_t)f32_to_bf16_rne(v[e]);
          }
        }
    }
  }
}

}  // namespace

hipError_t launch_q4k_mmq(const void *act_q8, const void *w, void *out, int32_t *dots,
                          uint32_t m0, uint32_t mt, uint32_t n0, uint32_t nt, uint32_t m,
                          uint32_t n, uint32_t k, hipStream_t s) {
  if (dots == nullptr) {
    const dim3 grid((n + BN - 1) / BN, (m + BM - 1) / BM);
    hipLaunchKernelGGL(q4k_mmq_kernel<false>, grid, dim3(kThreads), 0, s,
                       static_cast<const uint8_t *>(act_q8), static_cast<const uint8_t *>(w),
                       static_cast<uint16_t *>(out), nullptr, m, n, k, 0u, 0u, 0u, 0u, 0u, 0u);
  } else {
    const uint32_t tn0 = n0 / BN, tn1 = (n0 + nt - 1) / BN;
    const uint32_t tm0 = m0 / BM, tm1 = (m0 + mt - 1) / BM;
    const dim3 grid(tn1 - tn0 + 1, tm1 - tm0 + 1);
    hipLaunchKernelGGL(q4k_mmq_kernel<true>, grid, dim3(kThreads), 0, s,
                       static_cast<const uint8_t *>(act_q8), static_cast<const uint8_t *>(w),
                       nullptr, dots, m, n, k, m0, mt, n0, nt, tn0, tm0);
  }
  return hipGetLastError();
}

}  // namespace bqmm

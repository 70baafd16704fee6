// Q2_0 x q8_1 MMQ on CDNA4 int8 matrix cores.
//
// [page layers/qwen3_ssm/init_q2.rs, fn qkvz_q2_prefill_gemm: out[m, n] =
//  input[m, k] @ W^T through quantize_act_q8_1 and q2_0_mmq_gemm, group 128;
//  fn set_packed_q2_qkvz names the kernels q2_0_mmq128_{nc,wc}.]
//
// out[m][n] = sum_g dw[n][g] * sum_{b in g} da[m][b] * D[m][n][b],
//   D[m][n][b] = sum_{t<32} (c - 2) * q   (exact int32, one 32-block).
//
// Tile 128 (n) x 128 (m), 256 lanes = 4 waves of 64 (n) x 64 (m).  Per
// 128-wide k group the workgroup stages into LDS:
//   * the q8_1 codes of its 128 rows (int8, 128 B per row),
//   * the packed 2-bit codes of its 128 weight rows, unpacked once to signed
//     int8 (c - 2) with a byte-permute lookup,
//   * the group's weight scales (fp32) and, per activation row and block, an
//     integer multiplier mu = da * 2^(30 - E) where E is the binary16
//     exponent of the row's largest scale (exact whenever the block's scale
//     is within 2^5 of the row maximum; otherwise rounded to 16 bits).
// Each wave then runs v_mfma_i32_32x32x32_i8 (K = 32 = one q8_1 block) with
// the weights as the A operand and the activations as B, so a lane's 16
// accumulators share one activation row: the activation multiplier is one
// lane value.  Per block: acc += mu * D (24-bit integer multiply-add, exact
// int32 accumulation over the 128-group); per group: out += dw * float(acc);
// at the end out *= 2^(E - 30) and is rounded to bf16.
#include "bqmm_internal.h"

namespace bqmm {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BN = 128;       // weight rows per tile
constexpr int BM = 128;       // activation rows per tile
constexpr int KG = 128;       // k per stage (one Q2_0 group = four q8_1 blocks)
constexpr int LDS_STRIDE = KG + 16;  // bytes per staged row; the pad spreads banks
constexpr int kThreads = 256;

__device__ __forceinline__ int mad_i24(int a, int b, int c) {
  // a, b fit in 24 bits (|D| <= 8128, mu < 2^16); one v_mad_i32_i24.
  return ((a << 8) >> 8) * ((b << 8) >> 8) + c;
}

// Signed code bytes (c - 2) of field j of a packed word: the field gives four
// 2-bit selectors, v_perm_b32 maps 0,1,2,3 -> 0xFE,0xFF,0x00,0x01.
__device__ __forceinline__ uint32_t unpack_signed(uint32_t word, int j) {
  const uint32_t sel = (word >> (2 * j)) & 0x03030303u;
  return __builtin_amdgcn_perm(0u, 0x0100FFFEu, sel);
}

template <bool kDump>
__global__ __launch_bounds__(kThreads) void q2_0_mmq_kernel(
    const uint8_t *__restrict__ act_q8, const uint8_t *__restrict__ w, uint16_t *__restrict__ out,
    int32_t *__restrict__ dots, uint32_t m, uint32_t n, uint32_t k, uint32_t m0, uint32_t mt,
    uint32_t n0, uint32_t nt, uint32_t tile_n0, uint32_t tile_m0) {
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint8_t w_lds[BN * LDS_STRIDE];
  __shared__ float dw_lds[BN];
  __shared__ int mu_lds[BM * 4];
  __shared__ int rowexp[BM];

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u;
  const uint32_t wave = tid >> 6;
  const uint32_t wn = wave & 1u, wm = wave >> 1;
  const uint32_t n_base = (blockIdx.x + tile_n0) * BN;
  const uint32_t m_base = (blockIdx.y + tile_m0) * BM;
  const uint32_t kpad = (k + 255u) / 256u * 256u;
  const uint32_t nblk_pad = kpad / 32u;
  const uint32_t ngroups = k / KG;
  const uint8_t *ds = act_q8 + (uint64_t)m * kpad;
  const uint16_t *wscale = reinterpret_cast<const uint16_t *>(w + (uint64_t)n * k / 4u);

  // Row exponent: binary16 exponent field of the largest block scale of the row.
  {
    const uint32_t r = tid >> 1, part = tid & 1u;
    uint32_t mx = 0;
    if (m_base + r < m) {
      const uint32_t *pairs =
          reinterpret_cast<const uint32_t *>(ds) + (uint64_t)(m_base + r) * nblk_pad;
      const uint32_t nb = k / 32u;
      for (uint32_t b = part; b < nb; b += 2) mx = max(mx, pairs[b] & 0x7FFFu);
    }
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 1));
    if (part == 0) rowexp[r] = (int)(mx >> 10);
  }

  float acc_out[2][2][16];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_out[a][b][r] = 0.0f;

  const v16i zero16 = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

  for (uint32_t g = 0; g < ngroups; ++g) {
    __syncthreads();  // previous group fully consumed (and rowexp visible)
    // activation codes: 128 rows x 128 bytes, 16 bytes per load
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t c = tid + kThreads * i;
      const uint32_t r = c >> 3, col = (c & 7u) * 16u;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m_base + r < m)
        v = *reinterpret_cast<const uint4 *>(act_q8 + (uint64_t)(m_base + r) * kpad + g * KG + col);
      *reinterpret_cast<uint4 *>(a_lds + r * LDS_STRIDE + col) = v;
    }
    // weight codes: 128 rows x 32 bytes, unpacked to signed int8
    {
      const uint32_t r = tid >> 1, half = tid & 1u;
      uint4 p = make_uint4(0xAAAAAAAAu, 0xAAAAAAAAu, 0xAAAAAAAAu, 0xAAAAAAAAu);  // codes 2 -> 0
      if (n_base + r < n)
        p = *reinterpret_cast<const uint4 *>(w + (uint64_t)(n_base + r) * (k / 4u) + g * 32u + half * 16u);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 s = make_uint4(unpack_signed(p.x, j), unpack_signed(p.y, j),
                                   unpack_signed(p.z, j), unpack_signed(p.w, j));
        *reinterpret_cast<uint4 *>(w_lds + r * LDS_STRIDE + 32 * j + 16 * half) = s;
      }
    }
    if (tid < BN) {
      const uint32_t r = tid;
      dw_lds[r] = (n_base + r < n) ? f16_bits_to_f32(wscale[(uint64_t)(n_base + r) * ngroups + g]) : 0.0f;
    } else {
      const uint32_t r = tid - BN;
      int mu[4] = {0, 0, 0, 0};
      if (m_base + r < m) {
        const uint4 pr = *reinterpret_cast<const uint4 *>(ds + 4ull * ((uint64_t)(m_base + r) * nblk_pad + 4u * g));
        const uint32_t pv[4] = {pr.x, pr.y, pr.z, pr.w};
        const int e = rowexp[r];
#pragma unroll
        for (int b = 0; b < 4; ++b) mu[b] = (int)rintf(ldexpf(f16_bits_to_f32(pv[b] & 0xFFFFu), 30 - e));
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) mu_lds[r * 4 + b] = mu[b];
    }
    __syncthreads();

    int acc_int[2][2][16];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      v4i A[2], B[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        A[s] = *reinterpret_cast<const v4i *>(w_lds + (wn * 64 + s * 32 + (lane & 31)) * LDS_STRIDE + 32 * b + 16 * (lane >> 5));
        B[s] = *reinterpret_cast<const v4i *>(a_lds + (wm * 64 + s * 32 + (lane & 31)) * LDS_STRIDE + 32 * b + 16 * (lane >> 5));
      }
#pragma unroll
      for (int sn = 0; sn < 2; ++sn)
#pragma unroll
        for (int sm = 0; sm < 2; ++sm) {
          const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[sn], B[sm], zero16, 0, 0, 0);
          if constexpr (kDump) {
            const uint32_t mm = m_base + wm * 64 + sm * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const uint32_t nn = n_base + wn * 64 + sn * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
              if (mm >= m0 && mm < m0 + mt && nn >= n0 && nn < n0 + nt)
                dots[((uint64_t)(mm - m0) * nt + (nn - n0)) * (k / 32u) + 4u * g + b] = D[r];
            }
          } else {
            const int mu = mu_lds[(wm * 64 + sm * 32 + (lane & 31)) * 4 + b];
#pragma unroll
            for (int r = 0; r < 16; ++r)
              acc_int[sn][sm][r] = mad_i24(D[r], mu, b == 0 ? 0 : acc_int[sn][sm][r]);
          }
        }
    }
    if constexpr (!kDump) {
#pragma unroll
      for (int sn = 0; sn < 2; ++sn) {
        float dwv[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 t = *reinterpret_cast<const float4 *>(dw_lds + wn * 64 + sn * 32 + 8 * q + 4 * (lane >> 5));
          dwv[4 * q + 0] = t.x; dwv[4 * q + 1] = t.y; dwv[4 * q + 2] = t.z; dwv[4 * q + 3] = t.w;
        }
#pragma unroll
        for (int sm = 0; sm < 2; ++sm)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            acc_out[sn][sm][r] = fmaf((float)acc_int[sn][sm][r], dwv[r], acc_out[sn][sm][r]);
      }
    }
  }

  if constexpr (!kDump) {
    const bool vec = (n % 4u) == 0u;
#pragma unroll
    for (int sm = 0; sm < 2; ++sm) {
      const uint32_t mloc = wm * 64 + sm * 32 + (lane & 31);
      const uint32_t mm = m_base + mloc;
      if (mm >= m) continue;
      const float scale = ldexpf(1.0f, rowexp[mloc] - 30);
      uint16_t *orow = out + (uint64_t)mm * n;
#pragma unroll
      for (int sn = 0; sn < 2; ++sn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t nn = n_base + wn * 64 + sn * 32 + 8 * q + 4 * (lane >> 5);
          const float *v = &acc_out[sn][sm][4 * q];
          if (vec && nn + 4 <= n) {
            *reinterpret_cast<uint2 *>(orow + nn) =
                make_uint2(pack_bf16x2(v[0] * scale, v[1] * scale), pack_bf16x2(v[2] * scale, v[3] * scale));
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (nn + e < n) orow[nn + e] = (uint16_t)f32_to_bf16_rne(v[e] * scale);
          }
        }
    }
  }
}

}  // namespace

hipError_t launch_q2_0_mmq(const void *act_q8, const void *w, void *out, int32_t *dots,
                           uint32_t m0, uint32_t mt, uint32_t n0, uint32_t nt, uint32_t m,
                           uint32_t n, uint32_t k, hipStream_t s) {
  if (dots == nullptr) {
    const dim3 grid((n + BN - 1) / BN, (m + BM - 1) / BM);
    hipLaunchKernelGGL(q2_0_mmq_kernel<false>, grid, dim3(kThreads), 0, s,
                       static_cast<const uint8_t *>(act_q8), static_cast<const uint8_t *>(w),
                       static_cast<uint16_t *>(out), nullptr, m, n, k, 0u, 0u, 0u, 0u, 0u, 0u);
  } else {
    const uint32_t tn0 = n0 / BN, tn1 = (n0 + nt - 1) / BN;
    const uint32_t tm0 = m0 / BM, tm1 = (m0 + mt - 1) / BM;
    const dim3 grid(tn1 - tn0 + 1, tm1 - tm0 + 1);
    hipLaunchKernelGGL(q2_0_mmq_kernel<true>, grid, dim3(kThreads), 0, s,
                       static_cast<const uint8_t *>(act_q8), static_cast<const uint8_t *>(w),
                       nullptr, dots, m, n, k, m0, mt, n0, nt, tn0, tm0);
  }
  return hipGetLastError();
}

}  // namespace bqmm

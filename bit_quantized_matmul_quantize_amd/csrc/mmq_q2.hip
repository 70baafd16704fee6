// Q2_0 x q8_1 MMQ on CDNA4 int8 matrix cores.
//
// [page layers/qwen3_ssm/init_q2.rs, fn qkvz_q2_prefill_gemm: out[m, n] =
//  input[m, k] @ W^T through quantize_act_q8_1 and q2_0_mmq_gemm, group 128;
//  fn set_packed_q2_qkvz names the kernels q2_0_mmq128_{nc,wc}.]
//
// out[m][n] = sum_g dw[n][g] * sum_{b in g} da[m][b] * D[m][n][b],
//   D[m][n][b] = sum_{t<32} (c - 2) * q   (exact int32, one 32-block).
//
// Tile BN (n) x 128 (m), 256 lanes = 4 waves, each of TN x TM 32 x 32
// subtiles: 128 x 128 (waves of 64 x 64) by default, and 96 x 128 (waves of
// 96 x 32) where that fills the chip in fewer rounds of workgroups.  Per
// 128-wide k group the workgroup stages into LDS:
//   * the q8_1 codes of its 128 rows (int8, 128 B per row),
//   * the packed 2-bit codes of its BN weight rows, unpacked once to signed
//     int8 (c - 2) with a byte-permute lookup,
//   * the group's weight scales (fp32) and, per activation row and block, an
//     integer multiplier mu = da * 2^(30 - E) where E is the binary16
//     exponent of the row's largest scale.
// Each wave then runs v_mfma_i32_32x32x32_i8 (K = 32 = one q8_1 block) with
// the weights as the A operand and the activations as B, so a lane's 16
// accumulators share one activation row: the activation multiplier is one
// lane value.  Per block: acc += mu * D (24-bit integer multiply-add, exact
// int32 accumulation over the 128-group); per group: out += dw * float(acc);
// at the end out *= 2^(E - 30) and is rounded to bf16.
//
// mu is exact when the block's binary16 exponent is at most 5 below E: the
// 11-bit significand shifted left by at most 5 stays below 2^16, and four
// products of |D| <= 8128 with it fit int32.  A block exactly 6 below gets
// its significand halved and rounded to nearest: its scale is applied with a
// relative error of at most 2^-10 (twice the binary16 rounding d itself
// carried), no more.  The workloads' rows stay within that span of 6 (with
// 1% outlier channels about 3% of rows reach it).  For a row whose nonzero
// block scales spread wider, the tile runs the k loop once per band of seven
// exponents: pass p takes E_p = E - 7p, gives mu = da * 2^(30 - E_p) to the
// blocks whose exponent lies in [E_p - 6, E_p] and 0 to every other block,
// and carries the factor 2^-7p in the staged weight scales, so the passes add
// up to the whole product and no block's scale is rounded by more than the
// above or dropped (at most five passes cover the binary16 range).  A
// subnormal scale takes exponent 0 here: the bands that hold 0 have E_p <= 6,
// where its multiplier is an exact integer.  The
// prologue finds the number of passes; a tile of rows within the span takes
// one.
#include "bqmm_internal.h"

namespace bqmm {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 128;       // activation rows per tile
constexpr int KG = 128;       // k per stage (one Q2_0 group = four q8_1 blocks)
constexpr int LDS_STRIDE = KG + 16;  // bytes per staged row; the pad spreads banks
constexpr int kThreads = 256;
constexpr int kActBytes = BM * LDS_STRIDE;
// one LDS stage: activation codes, unpacked weight codes, weight scales, multipliers
__host__ __device__ constexpr int stage_bytes(int bn) { return kActBytes + bn * LDS_STRIDE + bn * 4 + BM * 16; }

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

// Exponent field of a binary16 scale (low 16 bits of h), at least 1: the
// field of a row's largest scale sets its top band (a subnormal top scale is
// scaled like field 1's).
__device__ __forceinline__ uint32_t exp_field(uint32_t h) { return max((h >> 10) & 31u, 1u); }

// The band position of a block scale: its exponent field, 0 for a subnormal,
// whose value d = f * 2^-24 gives the integer f * 2^(6 - ep) in every band
// that holds field 0 (ep <= 6), so subnormal scales are never rounded.
__device__ __forceinline__ uint32_t band_field(uint32_t h) { return (h >> 10) & 31u; }

// Integer multiplier of block scale h in the pass whose top exponent is ep:
// da * 2^(30 - ep) when the block's band position lies in [ep - 6, ep],
// else 0 (a zero scale gives 0 either way).
__device__ __forceinline__ int band_mu(uint32_t h, int ep) {
  const float v = ldexpf(f16_bits_to_f32(h & 0xFFFFu), 30 - ep);
  return (uint32_t)(ep - (int)band_field(h)) <= 6u ? (int)rintf(v) : 0;
}

// TN x TM subtiles of 32 x 32 per wave, WN waves along n (4 / WN along m).
template <bool kDump, int TN, int TM, int WN>
__global__ __launch_bounds__(kThreads, kDump ? 1 : 2) void q2_0_mmq_kernel(
    const uint8_t *__restrict__ act_q8, const uint8_t *__restrict__ w, uint16_t *__restrict__ out,
    int32_t *__restrict__ dots, uint32_t m, uint32_t n, uint32_t k, uint32_t m0, uint32_t mt,
    uint32_t n0, uint32_t nt, uint32_t tile_n0, uint32_t tile_m0, uint32_t ldc) {
  constexpr int WM = 4 / WN;
  constexpr int BN = 32 * TN * WN;
  static_assert(WN * WM == 4 && 32 * TM * WM == BM, "four waves cover 128 activation rows");
  static_assert(2 * BN <= kThreads && BN + BM <= kThreads, "one staging thread per 16 weight bytes and per scale row");
  constexpr int kWBytes = BN * LDS_STRIDE;
  constexpr int kStageBytes = stage_bytes(BN);
  constexpr int kSteps = 4 * TN * TM;  // (n-subtile, m-subtile, block) per group
  // Two LDS stages (dynamic shared memory, kStageBytes each): group g is
  // computed from stage g % 2 while group g + 1 is written into the other.
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  // Per tile row: the binary16 exponent field E of its largest block scale.
  __shared__ int mmq_rowexp[BM];
  // Passes of the k loop the tile needs (one per band of seven exponents).
  __shared__ int mmq_passes;

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u, l32 = lane & 31u, hi = lane >> 5;
  const uint32_t wave = tid >> 6;
  const uint32_t wn = wave % WN, wm = wave / WN;
  const uint32_t n_base = (blockIdx.x + tile_n0) * BN;
  const uint32_t m_base = (blockIdx.y + tile_m0) * BM;
  const uint32_t kpad = (k + 255u) / 256u * 256u;
  const uint32_t nblk_pad = kpad / 32u;
  const uint32_t ngroups = k / KG;
  const uint8_t *ds = act_q8 + (uint64_t)m * kpad;
  const uint16_t *wscale = reinterpret_cast<const uint16_t *>(w + (uint64_t)n * k / 4u);

  // Global -> register staging.  Rows past m or n read the last valid row
  // (no branch around the loads); their results are never stored.  Threads
  // beyond the 2 BN weight loaders and the BN + BM scale loaders load a
  // valid row too and skip the LDS write.
  const uint32_t a_row[4] = {min(m_base + (tid >> 3), m - 1u), min(m_base + 32u + (tid >> 3), m - 1u),
                             min(m_base + 64u + (tid >> 3), m - 1u), min(m_base + 96u + (tid >> 3), m - 1u)};
  const uint32_t a_col = (tid & 7u) * 16u;
  const bool w_stager = (2 * BN == kThreads) || tid < 2u * BN;
  const bool s_stager = (BN + BM == kThreads) || tid < (uint32_t)(BN + BM);
  const uint32_t w_row = min(n_base + (w_stager ? tid >> 1 : 0u), n - 1u), w_half = tid & 1u;
  const uint32_t s_row = (tid < BN) ? min(n_base + tid, n - 1u) : min(m_base + (s_stager ? tid - BN : 0u), m - 1u);

  // Row exponent: exponent field E (exp_field) of the largest block scale of
  // the row, and the smallest band position among its nonzero block scales
  // (0 for a subnormal), which give the row's band passes (E - min) / 7 + 1; the tile takes the most of
  // its rows.  Two lanes per row read its (d, s) pairs as 16-byte chunks of four
  // blocks (k % 128 == 0, so the row holds whole chunks), eight loads in
  // flight per batch: one memory round trip per batch instead of one per
  // block.  Chunk indices past the row's end are clamped to its last chunk,
  // which leaves both extremes unchanged.
  if (tid == 0) mmq_passes = 1;
  {
    const uint32_t r = tid >> 1, part = tid & 1u;
    const uint4 *chunks =
        reinterpret_cast<const uint4 *>(ds + 4ull * (uint64_t)min(m_base + r, m - 1u) * nblk_pad);
    const uint32_t nq = k / 128u;
    uint32_t mx = 0, mn = 31u;
    // band position of a nonzero scale; 31, above every field, for a zero one
    auto nz_field = [](uint32_t h) { return (h & 0x7FFFu) == 0u ? 31u : band_field(h); };
    for (uint32_t c0 = part; c0 < nq; c0 += 16u) {
      uint4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = chunks[min(c0 + 2u * j, nq - 1u)];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        mx = max(mx, max(max(v[j].x & 0x7FFFu, v[j].y & 0x7FFFu), max(v[j].z & 0x7FFFu, v[j].w & 0x7FFFu)));
        mn = min(mn, min(min(nz_field(v[j].x), nz_field(v[j].y)), min(nz_field(v[j].z), nz_field(v[j].w))));
      }
    }
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 1));
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, 1));
    __syncthreads();  // mmq_passes initialised
    if (part == 0) {
      const int e = (int)exp_field(mx);
      mmq_rowexp[r] = e;
      if ((int)mn < e - 6) atomicMax(&mmq_passes, (e - (int)mn) / 7 + 1);
    }
  }
  __syncthreads();  // mmq_rowexp and mmq_passes visible

  // Prefetch registers for one group (next group's data is in flight while
  // the current group computes).
  uint4 ra0, ra1, ra2, ra3, rw, rds = make_uint4(0, 0, 0, 0);
  uint32_t rs16 = 0;
#define BQMM_FETCH(g)                                                                                   \
  do {                                                                                                  \
    ra0 = *reinterpret_cast<const uint4 *>(act_q8 + (uint64_t)a_row[0] * kpad + (g) * KG + a_col);       \
    ra1 = *reinterpret_cast<const uint4 *>(act_q8 + (uint64_t)a_row[1] * kpad + (g) * KG + a_col);       \
    ra2 = *reinterpret_cast<const uint4 *>(act_q8 + (uint64_t)a_row[2] * kpad + (g) * KG + a_col);       \
    ra3 = *reinterpret_cast<const uint4 *>(act_q8 + (uint64_t)a_row[3] * kpad + (g) * KG + a_col);       \
    rw = *reinterpret_cast<const uint4 *>(w + (uint64_t)w_row * (k / 4u) + (g) * 32u + w_half * 16u);    \
    if (tid < BN)                                                                                       \
      rs16 = wscale[(uint64_t)s_row * ngroups + (g)];                                                   \
    else                                                                                                \
      rds = *reinterpret_cast<const uint4 *>(ds + 4ull * ((uint64_t)s_row * nblk_pad + 4u * (g)));     \
  } while (0)

  float acc_out[TN][TM][16];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_out[a][b][r] = 0.0f;

  const v16i zero16 = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

  // Write the prefetched group into LDS stage `st`, for band pass `pass`.
#define BQMM_STAGE(st, pass)                                                                                 \
  do {                                                                                                   \
    uint8_t *a_lds = lds + (st) * kStageBytes;                                                           \
    uint8_t *w_lds = a_lds + kActBytes;                                                                  \
    float *dw_lds = reinterpret_cast<float *>(w_lds + kWBytes);                                          \
    int *mu_lds = reinterpret_cast<int *>(dw_lds + BN);                                                  \
    *reinterpret_cast<uint4 *>(a_lds + (0 * 32 + (tid >> 3)) * LDS_STRIDE + a_col) = ra0;                \
    *reinterpret_cast<uint4 *>(a_lds + (1 * 32 + (tid >> 3)) * LDS_STRIDE + a_col) = ra1;                \
    *reinterpret_cast<uint4 *>(a_lds + (2 * 32 + (tid >> 3)) * LDS_STRIDE + a_col) = ra2;                \
    *reinterpret_cast<uint4 *>(a_lds + (3 * 32 + (tid >> 3)) * LDS_STRIDE + a_col) = ra3;                \
    if (w_stager) {                                                                                      \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                                    \
        const uint4 sv = make_uint4(unpack_signed(rw.x, j), unpack_signed(rw.y, j),                      \
                                    unpack_signed(rw.z, j), unpack_signed(rw.w, j));                     \
        *reinterpret_cast<uint4 *>(w_lds + (tid >> 1) * LDS_STRIDE + 32 * j + 16 * w_half) = sv;         \
      }                                                                                                  \
    }                                                                                                    \
    if (tid < BN) {                                                                                      \
      dw_lds[tid] = ldexpf(f16_bits_to_f32(rs16), -7 * (int)(pass));                                     \
    } else if (s_stager) {                                                                               \
      const int ep = mmq_rowexp[tid - BN] - 7 * (int)(pass);                                             \
      const int4 mu = make_int4(band_mu(rds.x, ep), band_mu(rds.y, ep), band_mu(rds.z, ep),              \
                                band_mu(rds.w, ep));                                                     \
      *reinterpret_cast<int4 *>(mu_lds + (tid - BN) * 4) = mu;                                           \
    }                                                                                                    \
  } while (0)

  // Group stream: step t computes group t % ngroups of pass t / ngroups (one
  // pass for a tile of ordinary rows).  (g, p) is the group and pass of step
  // t, (g1, p1) of step t + 1, (g2, p2) of step t + 2, advanced without
  // division.
  const uint32_t passes = kDump ? 1u : __builtin_amdgcn_readfirstlane(mmq_passes);
  const uint32_t nsteps = ngroups * passes;
  uint32_t g = 0, g1 = 0, p1 = 0, g2 = 0, p2 = 0;
  auto next = [ngroups](uint32_t &gg, uint32_t &pp) {
    if (++gg == ngroups) {
      gg = 0;
      ++pp;
    }
  };
  next(g1, p1);
  g2 = g1;
  p2 = p1;
  next(g2, p2);
  BQMM_FETCH(0u);
  BQMM_STAGE(0, 0u);
  if (nsteps > 1) BQMM_FETCH(g1);
  // Loop body: one barrier, then stage step t + 1 into the other LDS stage and
  // start the loads of step t + 2, then compute step t.  The barrier both
  // publishes stage t and guarantees that every wave has finished reading the
  // stage about to be overwritten (it held step t - 1).  The compute is last
  // in the body: placed before a barrier, its epilogue gets sunk below it and
  // all MFMA results of a group stay alive across the barrier.
  for (uint32_t t = 0; t < nsteps; ++t, g = g1, g1 = g2, p1 = p2, next(g2, p2)) {
    __syncthreads();
    if (t + 1 < nsteps) {
      BQMM_STAGE((t + 1) & 1u, p1);
      if (t + 2 < nsteps) BQMM_FETCH(g2);
    }
    const uint8_t *a_lds = lds + (t & 1u) * kStageBytes;
    const uint8_t *w_lds = a_lds + kActBytes;
    const float *dw_lds = reinterpret_cast<const float *>(w_lds + kWBytes);
    const int *mu_lds = reinterpret_cast<const int *>(dw_lds + BN);

    // Operands of the group: both n-subtiles (weights, A) and both m-subtiles
    // (activations, B) for the four blocks, and the activation multipliers.
    v4i A[TN][4], B[TM][4];
    int mu[TM][4];
#pragma unroll
    for (int sm = 0; sm < TM; ++sm) {
      const uint32_t ml = wm * (32 * TM) + sm * 32 + l32;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        B[sm][b] = *reinterpret_cast<const v4i *>(a_lds + ml * LDS_STRIDE + 32 * b + 16 * hi);
      const int4 t = *reinterpret_cast<const int4 *>(mu_lds + ml * 4);
      mu[sm][0] = t.x; mu[sm][1] = t.y; mu[sm][2] = t.z; mu[sm][3] = t.w;
    }
#pragma unroll
    for (int sn = 0; sn < TN; ++sn) {
      const uint32_t nl = wn * (32 * TN) + sn * 32 + l32;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        A[sn][b] = *reinterpret_cast<const v4i *>(w_lds + nl * LDS_STRIDE + 32 * b + 16 * hi);
    }

    // In the 96 x 128 layout the wave computing a group takes issue priority
    // over the wave of the other workgroup on its SIMD (which is staging or
    // waiting): 5% faster at m = 512.  On the 128 x 128 layout it measured
    // the same at m = 2048 and 1-3% slower on the FFN shapes, so it is off.
    constexpr bool kPrio = TM == 1;
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
    // kSteps steps (sn, sm, b), software-pipelined by one: the MFMA of step i + 1
    // is issued before the epilogue of step i, so the matrix core runs while
    // the VALU folds the previous block; two result registers alternate.  A
    // scheduling barrier after each step keeps the compiler from clustering
    // the MFMAs (which would keep all 16 results alive).
    v16i D[2];
    int acc[16];
    float dwv[16];
#pragma unroll
    for (int i = 0; i <= kSteps; ++i) {
      if (i < kSteps) {
        const int sn = i / (4 * TM), sm = (i / 4) % TM, b = i & 3;
        D[i & 1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[sn][b], B[sm][b], zero16, 0, 0, 0);
        // issue the MFMA ahead of the previous step's epilogue: left to itself
        // the scheduler can sink it below, and the next step then waits for
        // the result (a run of s_nop hazard padding at every such step)
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i > 0) {
        const int p = i - 1;
        const int sn = p / (4 * TM), sm = (p / 4) % TM, b = p & 3;
        const v16i &Dp = D[p & 1];
        if constexpr (kDump) {
          const uint32_t mm = m_base + wm * (32 * TM) + sm * 32 + l32;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t nn = n_base + wn * (32 * TN) + sn * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (mm >= m0 && mm < m0 + mt && nn >= n0 && nn < n0 + nt)
              dots[((uint64_t)(mm - m0) * nt + (nn - n0)) * (k / 32u) + 4u * g + b] = Dp[r];
          }
        } else {
          if (p % (4 * TM) == 0) {
            // weight scales of n-subtile sn: loaded at its first step, after the
            // last flush of the previous n-subtile, three steps before first use
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float4 t = *reinterpret_cast<const float4 *>(dw_lds + wn * (32 * TN) + sn * 32 + 8 * q + 4 * hi);
              dwv[4 * q + 0] = t.x; dwv[4 * q + 1] = t.y; dwv[4 * q + 2] = t.z; dwv[4 * q + 3] = t.w;
            }
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] = mad_i24(Dp[r], mu[sm][b], b == 0 ? 0 : acc[r]);
          if (b == 3) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
              acc_out[sn][sm][r] = fmaf((float)acc[r], dwv[r], acc_out[sn][sm][r]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
  }
#undef BQMM_FETCH
#undef BQMM_STAGE

  if constexpr (!kDump) {
    const bool full = (m_base + BM <= m) && (n_base + BN <= n) && (ldc % 4u) == 0u;
#pragma unroll
    for (int sm = 0; sm < TM; ++sm) {
      const uint32_t mloc = wm * (32 * TM) + sm * 32 + l32;
      const uint32_t mm = m_base + mloc;
      const float scale = ldexpf(1.0f, mmq_rowexp[mloc] - 30);
      uint16_t *orow = out + (uint64_t)min(mm, m - 1u) * ldc;
#pragma unroll
      for (int sn = 0; sn < TN; ++sn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t nn = n_base + wn * (32 * TN) + sn * 32 + 8 * q + 4 * hi;
          const float *v = &acc_out[sn][sm][4 * q];
          if (full) {
            *reinterpret_cast<uint2 *>(orow + nn) =
                make_uint2(pack_bf16x2(v[0] * scale, v[1] * scale), pack_bf16x2(v[2] * scale, v[3] * scale));
          } else if (mm < m) {
            if ((ldc % 4u) == 0u && nn + 4 <= n) {
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
}

template <int TN, int TM, int WN>
hipError_t launch_mmq_layout(const void *act_q8, const void *w, void *out, uint32_t m, uint32_t n, uint32_t k,
                             uint32_t ldc, hipStream_t s) {
  constexpr int BN = 32 * TN * WN;
  constexpr int lds = 2 * stage_bytes(BN);
  // Two stages exceed the 64 KB default dynamic-LDS limit; gfx950 allows 160 KB.
  const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void *>(q2_0_mmq_kernel<false, TN, TM, WN>), lds);
  if (e != hipSuccess) return e;
  const dim3 grid((uint32_t)(((uint64_t)n + BN - 1) / BN), (uint32_t)(((uint64_t)m + BM - 1) / BM));
  hipLaunchKernelGGL((q2_0_mmq_kernel<false, TN, TM, WN>), grid, dim3(kThreads), lds, s,
                     static_cast<const uint8_t *>(act_q8), static_cast<const uint8_t *>(w),
                     static_cast<uint16_t *>(out), nullptr, m, n, k, 0u, 0u, 0u, 0u, 0u, 0u, ldc);
  return hipGetLastError();
}

}  // namespace

// The tile is chosen by how many rounds of resident workgroups (two per CU)
// the grid takes: a 96 x 128 tile holds 3/4 of a 128 x 128 tile's work, so
// it wins where it needs fewer than 4/3 as many rounds.  For m = 512,
// n = 12288 on 256 CUs: 384 large tiles leave a quarter of the 512 slots
// empty (one round), 512 small tiles fill them (one round of 3/4 the time).
hipError_t launch_q2_0_mmq(const void *act_q8, const void *w, void *out, int32_t *dots,
                           uint32_t m0, uint32_t mt, uint32_t n0, uint32_t nt, uint32_t m,
                           uint32_t n, uint32_t k, uint32_t ldc, hipStream_t s) {
  if (dots == nullptr) {
    int cus = 0;
    const hipError_t e = device_cu_count(&cus);
    if (e != hipSuccess) return e;
    const uint64_t slots = 2ull * (uint64_t)(cus > 0 ? cus : 1);
    const uint64_t tiles_m = ((uint64_t)m + BM - 1) / BM;
    const uint64_t rounds128 = ((n + 127ull) / 128ull * tiles_m + slots - 1) / slots;
    const uint64_t rounds96 = ((n + 95ull) / 96ull * tiles_m + slots - 1) / slots;
    if (3 * rounds96 < 4 * rounds128) return launch_mmq_layout<3, 1, 1>(act_q8, w, out, m, n, k, ldc, s);
    return launch_mmq_layout<2, 2, 2>(act_q8, w, out, m, n, k, ldc, s);
  }
  // Block dots of a window: the 128 x 128 layout.
  constexpr int BN = 128;
  constexpr int lds = 2 * stage_bytes(BN);
  const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void *>(q2_0_mmq_kernel<true, 2, 2, 2>), lds);
  if (e != hipSuccess) return e;
  const uint32_t tn0 = n0 / BN, tn1 = (n0 + nt - 1) / BN;
  const uint32_t tm0 = m0 / BM, tm1 = (m0 + mt - 1) / BM;
  const dim3 grid(tn1 - tn0 + 1, tm1 - tm0 + 1);
  hipLaunchKernelGGL((q2_0_mmq_kernel<true, 2, 2, 2>), grid, dim3(kThreads), lds, s,
                     static_cast<const uint8_t *>(act_q8), static_cast<const uint8_t *>(w), nullptr, dots, m, n,
                     k, m0, mt, n0, nt, tn0, tm0, n);
  return hipGetLastError();
}

}  // namespace bqmm

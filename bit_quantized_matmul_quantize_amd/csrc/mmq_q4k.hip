// Q4_K x q8_1 MMQ on CDNA4 matrix cores.
//
// [page layers/ops/q4k_mmq.rs, fn q4k_mmq_gemm: C[m, n] = A[m, k] x W[n, k]
//  with A in q8_1 and W in block_q4_K (256 weights in 144 bytes), BF16 store,
//  any n (a with-check variant for n % 128 != 0).]
//
// out[m][n] = sum_sb d[n] * sum_j da[m][j] * sc_j[n] * D[m][n][j]
//             - sum_j dmin[n]*m_j[n] * s[m][j]
//   D = sum_{t<32} q4 * q (exact, one 32-block),  s = the stored q8_1 sum (da * sum q).
//
// The weight's 6-bit sub-scale is moved onto the matrix core: the weight
// operand is q4 * sc_j, an exact small integer in binary16 (<= 945).  The
// activation scale is moved into the other operand: it is
// q * da * 2^-e rounded once to binary16, where 2^e is a power of two per
// activation row, chosen by a prologue from the row's largest da (the
// exponent field f of that da, at least 1, gives e = f - 23, so that
// |q * da * 2^-e| < 127 * 2^9 < 65504 and da * 2^-e is exact for blocks
// within 2^22 of the largest; a block further below loses one bit of its
// scale per binade and, beyond about 2^33, all of it).
// v_mfma_f32_32x32x16_f16 then accumulates a whole super-block in place
// (fp32, its first MFMA starting from zero), and per super-block and output
// two fmas remain: one with the weight row's d and one with the min term.
// The min term runs on the matrix core too, once per super-block:
// v_mfma_f32_32x32x8_f16 with A = m_j (exact small integers) for the eight
// sub-blocks and B = their stored sums s times 2^-(e + 6) (exact, and below
// 2^15) gives sum_j m_j * s_j * 2^-(e + 6), and one fma per output applies
// -64 dmin.  (Folding dmin into A would round dmin * m_j to binary16 and
// overflow it for dmin above 1040, inside the format's range.)  2^e is
// applied once, when the outputs are stored.  Rounding the activation operand
// costs a relative 2^-11 per value, below the 2^-8 that q8_1 codes carry; in
// exchange the kernel issues 11.7 instead of 19.1 VALU instructions per
// MFMA (SQ counters), which made it about 9% faster: on this kernel the staging (global
// loads, conversion, LDS writes), the barriers and the flush each take a
// share of the time, and a copy without any MFMA still ran 87% as long.
//
// Tile 128 (n) x 128 (m), 256 lanes = 4 waves of 64 (n) x 64 (m), two
// workgroups per CU (76,288 bytes of LDS each); k is staged 64 at a time
// (one 64-weight chunk of a super-block: sub-block 2t in the low nibbles,
// 2t + 1 in the high nibbles of the same 32 bytes) through two LDS stages,
// both operands converted to binary16 once per workgroup while they are
// written: the q8_1 codes by an exponent-bias trick (bytes xor 0x80 under the
// exponent of 1024, then one packed subtraction of 1152) and one packed
// multiply by da * 2^-e, the 4-bit codes likewise times sc_j with one packed
// fma.  Staged rows are 128 bytes with their 16-byte chunks XOR-swizzled by
// the row's low bits instead of padded, which lets two workgroups share a CU.
// (A 256 (m) x 128 (n) tile of eight waves, one workgroup per CU, measured
// 1-9% slower; so did splitting the eight waves into four that stage and four
// that compute, and 16 x 16 x 32 MFMA subtiles, which run at half the
// 32 x 32 x 16 rate here.  Unrolling the loop by a super-block, with and
// without a forced MFMA/VALU interleave of 4 to 9 VALU instructions per MFMA,
// and a swizzle by the row's bits 1-3 measured within 3% of this loop.)  The
// compute is last in the loop body (see the Q2_0 kernel for why).
#include "bqmm_internal.h"

namespace bqmm {
namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BN = 128;
constexpr int BM = 128;
constexpr int KS = 64;                       // k per stage: one chunk of a super-block
constexpr int ROW = 2 * KS;                  // bytes per staged binary16 row (16-byte chunks swizzled)
constexpr int kThreads = 256;
// one LDS stage
constexpr int kActBytes = BM * ROW;          // q * da * 2^-e, binary16
constexpr int kWBytes = BN * ROW;            // q4 * sc_j, binary16
constexpr int kStageBytes = kActBytes + kWBytes;
// per super-block (two of them, alternating): d of each weight row, the min
// term's weight operands m_j [BN][8] (binary16) and -dmin of each weight
// row (times 64), and the activation sums s * 2^-(e + 6) [BM][8]
constexpr int kSbD = 0;
constexpr int kSbNdmin = kSbD + BN * 4;
constexpr int kSbMin = kSbNdmin + BN * 4;
constexpr int kSbS = kSbMin + BN * 16;
constexpr int kSbBytes = kSbS + BM * 16;
constexpr int kLdsBytes = 2 * kStageBytes + 2 * kSbBytes;

// Byte offset of 16-byte chunk c of staged row r: the chunk index is XOR-ed
// with the row's low three bits, so eight consecutive rows read or written
// at one chunk index hit eight different bank groups (no padding needed).
__device__ __forceinline__ uint32_t swz(uint32_t r, uint32_t c) { return r * ROW + 16u * (c ^ (r & 7u)); }

__device__ __forceinline__ uint32_t sbyte(const uint32_t S[3], int i) { return (S[i >> 2] >> (8 * (i & 3))) & 0xFFu; }

__device__ __forceinline__ void scale_min(const uint32_t S[3], int j, uint32_t &sc, uint32_t &mn) {
  if (j < 4) {
    sc = sbyte(S, j) & 63u;
    mn = sbyte(S, j + 4) & 63u;
  } else {
    sc = (sbyte(S, j + 4) & 15u) | ((sbyte(S, j - 4) >> 6) << 4);
    mn = (sbyte(S, j + 4) >> 4) | ((sbyte(S, j) >> 6) << 4);
  }
}

// Four signed bytes of x as two pairs of binary16, exactly: xor 0x80 turns
// each byte into q + 128 (0..255); placed under the high byte 0x64 a half is
// 1024 + q + 128, and one packed subtraction of 1152 leaves q.
__device__ __forceinline__ void s8x4_to_f16(uint32_t x, uint32_t &lo, uint32_t &hi) {
  const uint32_t u = x ^ 0x80808080u;
  const v2h bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, u, 0x05010400u)) + bias);
  hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, u, 0x07030602u)) + bias);
}

// Four 4-bit codes (one per byte of x, already masked to 0..15) times sc, as
// two pairs of binary16: 1024 + q is exact under the exponent of 1024, and
// the packed fma (1024 + q) * sc - 1024 * sc is rounded once, from the exact
// q * sc <= 945, which binary16 holds exactly.
__device__ __forceinline__ void u4x4_to_f16(uint32_t x, v2h sc, v2h nsc1024, uint32_t &lo, uint32_t &hi) {
  const v2h a = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, x, 0x05010400u));
  const v2h b = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, x, 0x07030602u));
  lo = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(a, sc, nsc1024));
  hi = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(b, sc, nsc1024));
}

template <bool kDump>
__global__ __launch_bounds__(kThreads, 2) void q4k_mmq_kernel(
    const uint8_t *__restrict__ act_q8, const uint8_t *__restrict__ w, uint16_t *__restrict__ out,
    int32_t *__restrict__ dots, uint32_t m, uint32_t n, uint32_t k, uint32_t m0, uint32_t mt,
    uint32_t n0, uint32_t nt, uint32_t tile_n0, uint32_t tile_m0, uint32_t ldc) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  // exponent field ef of each tile row's largest activation block scale
  __shared__ int q4k_rowexp[BM];
  uint8_t *const sb_lds = lds + 2 * kStageBytes;

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63u, l32 = lane & 31u, hi = lane >> 5;
  const uint32_t wave = tid >> 6;
  const uint32_t wn = wave & 1u, wm = wave >> 1;  // wm in 0..1
  const uint32_t n_base = (blockIdx.x + tile_n0) * BN;
  const uint32_t m_base = (blockIdx.y + tile_m0) * BM;
  const uint32_t kpad = (k + 255u) / 256u * 256u;
  const uint32_t nblk_pad = kpad / 32u;
  const uint32_t nsb = k / 256u;
  const uint32_t nstages = k / KS;
  const uint8_t *ds = act_q8 + (uint64_t)m * kpad;

  // Global -> register staging; rows past m or n read the last valid row.
  //   activation codes: thread -> row tid / 2, bytes 32 * (tid % 2) of the stage;
  //   weight codes: thread -> row tid / 2, all 32 bytes of the chunk, of which
  //     it converts the low (tid % 2 = 0) or the high nibbles, plus its row's
  //     16-byte header (d, dmin, packed sub-scales/mins);
  //   activation (d, s): thread -> row tid / 2, block tid % 2 of the stage.
  const uint32_t srow = tid >> 1, sel = tid & 1u;
  const uint32_t a_row = min(m_base + srow, m - 1u);
  const uint32_t w_row = min(n_base + srow, n - 1u);
  uint4 ra0, ra1, rh, rw0, rw1;
  uint32_t rds;

  // Row exponent: the binary16 exponent field ef (at least 1) of the largest
  // q8_1 block scale of this thread's activation row; e = ef - 23.  The two
  // lanes of a row (tid ^ 1, same quad) scan alternate 16-byte chunks of four
  // (d, s) pairs, eight loads in flight per batch; chunk indices past the end
  // are clamped to the last chunk, which leaves the maximum unchanged.
  uint32_t ef = 1;
  if constexpr (!kDump) {
    const uint4 *chunks = reinterpret_cast<const uint4 *>(ds + 4ull * (uint64_t)a_row * nblk_pad);
    const uint32_t nq = k / 128u;
    uint32_t mx = 0;
    for (uint32_t c0 = sel; c0 < nq; c0 += 16u) {
      uint4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = chunks[min(c0 + 2u * j, nq - 1u)];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        mx = max(mx, max(max(v[j].x & 0x7FFFu, v[j].y & 0x7FFFu), max(v[j].z & 0x7FFFu, v[j].w & 0x7FFFu)));
    }
    mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0xB1, 0xF, 0xF, false));
    ef = max(mx >> 10, 1u);
    if (sel == 0u) q4k_rowexp[srow] = (int)ef;
  }
#define BQMM_FETCH(st)                                                                                  \
  do {                                                                                                  \
    const uint32_t sb_ = (st) >> 2, t_ = (st) & 3u;                                                     \
    const uint8_t *ap_ = act_q8 + (uint64_t)a_row * kpad + (st) * KS + 32u * sel;                      \
    ra0 = *reinterpret_cast<const uint4 *>(ap_);                                                        \
    ra1 = *reinterpret_cast<const uint4 *>(ap_ + 16);                                                   \
    const uint8_t *bp_ = w + ((uint64_t)w_row * nsb + sb_) * 144u;                                      \
    rh = *reinterpret_cast<const uint4 *>(bp_);                                                         \
    rw0 = *reinterpret_cast<const uint4 *>(bp_ + 16u + 32u * t_);                                       \
    rw1 = *reinterpret_cast<const uint4 *>(bp_ + 32u + 32u * t_);                                       \
    rds = *reinterpret_cast<const uint32_t *>(ds + 4ull * ((uint64_t)a_row * nblk_pad + 2u * (st) + sel)); \
  } while (0)

  // Write the prefetched stage into LDS stage buffer `buf`; stage st of
  // super-block st / 4 also writes that super-block's entries of the min
  // term and the activation sums (and, from its first stage, d).
#define BQMM_STAGE(buf, st)                                                                             \
  do {                                                                                                  \
    uint8_t *L = lds + (buf) * kStageBytes;                                                             \
    uint8_t *SB = sb_lds + (((st) >> 2) & 1u) * kSbBytes;                                               \
    const uint32_t t_ = (st) & 3u;                                                                      \
    {                                                                                                   \
      uint32_t h[16];                                                                                   \
      const uint32_t x_[8] = {ra0.x, ra0.y, ra0.z, ra0.w, ra1.x, ra1.y, ra1.z, ra1.w};                  \
      _Pragma("unroll") for (int i = 0; i < 8; ++i) s8x4_to_f16(x_[i], h[2 * i], h[2 * i + 1]);         \
      if (!kDump) {                                                                                     \
        const _Float16 a_ = (_Float16)__builtin_amdgcn_ldexpf(f16_bits_to_f32(rds & 0xFFFFu), 23 - (int)ef); \
        const v2h av_ = {a_, a_};                                                                       \
        _Pragma("unroll") for (int i = 0; i < 16; ++i)                                                  \
          h[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2h, h[i]) * av_);                     \
      }                                                                                                 \
      _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                     \
        *reinterpret_cast<uint4 *>(L + swz(srow, 4u * sel + i)) =                                       \
            make_uint4(h[4 * i], h[4 * i + 1], h[4 * i + 2], h[4 * i + 3]);                             \
    }                                                                                                   \
    {                                                                                                   \
      const uint32_t S_[3] = {rh.y, rh.z, rh.w};                                                        \
      uint32_t sc_, mn_;                                                                                \
      scale_min(S_, 2 * (int)t_ + (int)sel, sc_, mn_);                                                  \
      if (kDump) sc_ = 1u;                                                                              \
      const _Float16 f_ = (_Float16)(float)sc_;                                                         \
      const v2h s_ = {f_, f_};                                                                          \
      const v2h n_ = {(_Float16)(-1024.0f * (float)sc_), (_Float16)(-1024.0f * (float)sc_)};            \
      const uint32_t x_[8] = {rw0.x, rw0.y, rw0.z, rw0.w, rw1.x, rw1.y, rw1.z, rw1.w};                  \
      const uint32_t sh_ = 4u * sel;                                                                    \
      uint32_t o_[16];                                                                                  \
      _Pragma("unroll") for (int i = 0; i < 8; ++i)                                                     \
        u4x4_to_f16((x_[i] >> sh_) & 0x0F0F0F0Fu, s_, n_, o_[2 * i], o_[2 * i + 1]);                    \
      _Pragma("unroll") for (int i = 0; i < 4; ++i)                                                     \
        *reinterpret_cast<uint4 *>(L + kActBytes + swz(srow, 4u * sel + i)) =                           \
            make_uint4(o_[4 * i], o_[4 * i + 1], o_[4 * i + 2], o_[4 * i + 3]);                         \
      if (!kDump && t_ == 0u) {                                                                         \
        /* the two lanes of a row each write four of its eight min-term     */                          \
        /* operands (sub-blocks 2 sel, 2 sel + 1 and those plus 4, so that   */                         \
        /* each unpack form is known at compile time); both write d         */                          \
        const float d_ = f16_bits_to_f32(rh.x & 0xFFFFu), dmin_ = f16_bits_to_f32(rh.x >> 16);         \
        reinterpret_cast<float *>(SB + kSbD)[srow] = d_;                                                \
        reinterpret_cast<float *>(SB + kSbNdmin)[srow] = -64.0f * dmin_;                                \
        _Float16 *nm_ = reinterpret_cast<_Float16 *>(SB + kSbMin + srow * 16);                          \
        _Pragma("unroll") for (int q = 0; q < 2; ++q) {                                                 \
          const int j_ = 2 * (int)sel + q;                                                              \
          uint32_t sca_, mna_, scb_, mnb_;                                                              \
          scale_min(S_, j_, sca_, mna_);                                                                \
          scale_min(S_, j_ + 4, scb_, mnb_);                                                            \
          nm_[j_] = (_Float16)(float)mna_;                                                              \
          nm_[j_ + 4] = (_Float16)(float)mnb_;                                                          \
        }                                                                                               \
      }                                                                                                 \
    }                                                                                                   \
    reinterpret_cast<_Float16 *>(SB + kSbS)[8u * srow + 2u * t_ + sel] =                                \
        (_Float16)__builtin_amdgcn_ldexpf(f16_bits_to_f32(rds >> 16), 17 - (int)ef);                    \
  } while (0)

  v16f acc_out[2][2], acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_out[a][b][r] = 0.0f, acc[a][b][r] = 0.0f;
  const v16f zero16 = {};

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
    const uint32_t t = st & 3u;

    // Two blocks (sub-blocks 2t, 2t + 1), each two k-halves of 16 over the
    // four subtiles (sn: weights, A; sm: activations, B), accumulating the
    // super-block in place.
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      v8h A[2][2], B[2][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int sm = 0; sm < 2; ++sm)
          B[sm][h] = *reinterpret_cast<const v8h *>(a_lds + swz(wm * 64 + sm * 32 + l32, 4 * b + 2 * h + hi));
#pragma unroll
        for (int sn = 0; sn < 2; ++sn)
          A[sn][h] = *reinterpret_cast<const v8h *>(w_lds + swz(wn * 64 + sn * 32 + l32, 4 * b + 2 * h + hi));
      }
      // a super-block's first MFMA starts from zero (no clearing of acc)
      if (!kDump && b == 0 && t == 0u) {
#pragma unroll
        for (int sn = 0; sn < 2; ++sn)
#pragma unroll
          for (int sm = 0; sm < 2; ++sm)
            acc[sn][sm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[sn][0], B[sm][0], zero16, 0, 0, 0);
      } else {
#pragma unroll
        for (int sn = 0; sn < 2; ++sn)
#pragma unroll
          for (int sm = 0; sm < 2; ++sm)
            acc[sn][sm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[sn][0], B[sm][0], acc[sn][sm], 0, 0, 0);
      }
#pragma unroll
      for (int sn = 0; sn < 2; ++sn)
#pragma unroll
        for (int sm = 0; sm < 2; ++sm)
          acc[sn][sm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[sn][1], B[sm][1], acc[sn][sm], 0, 0, 0);
      if constexpr (kDump) {
#pragma unroll
        for (int sn = 0; sn < 2; ++sn)
#pragma unroll
          for (int sm = 0; sm < 2; ++sm) {
            const uint32_t mm = m_base + wm * 64 + sm * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const uint32_t nn = n_base + wn * 64 + sn * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
              if (mm >= m0 && mm < m0 + mt && nn >= n0 && nn < n0 + nt)
                dots[((uint64_t)(mm - m0) * nt + (nn - n0)) * (k / 32u) + 2u * st + b] = (int32_t)acc[sn][sm][r];
              acc[sn][sm][r] = 0.0f;
            }
          }
      }
    }

    if constexpr (!kDump) {
      if (t == 3u) {
        // end of a super-block: apply each weight row's d, then the min
        // term: sum_j m_j * s_j * 2^-(e + 6) on the matrix core (K = 8: the
        // super-block's eight sub-blocks) times -64 dmin
        const uint8_t *SB = sb_lds + ((st >> 2) & 1u) * kSbBytes;
#pragma unroll
        for (int sn = 0; sn < 2; ++sn) {
          float dv[16], nv[16];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t o = 4 * (wn * 64 + sn * 32 + 8 * q + 4 * hi);
            const float4 t4 = *reinterpret_cast<const float4 *>(SB + kSbD + o);
            const float4 u4 = *reinterpret_cast<const float4 *>(SB + kSbNdmin + o);
            dv[4 * q] = t4.x; dv[4 * q + 1] = t4.y; dv[4 * q + 2] = t4.z; dv[4 * q + 3] = t4.w;
            nv[4 * q] = u4.x; nv[4 * q + 1] = u4.y; nv[4 * q + 2] = u4.z; nv[4 * q + 3] = u4.w;
          }
          const uint32_t nl = wn * 64 + sn * 32 + l32;
          const v4h an = *reinterpret_cast<const v4h *>(SB + kSbMin + nl * 16 + 8 * hi);
#pragma unroll
          for (int sm = 0; sm < 2; ++sm) {
            const uint32_t ml = wm * 64 + sm * 32 + l32;
            const v4h bs = *reinterpret_cast<const v4h *>(SB + kSbS + ml * 16 + 8 * hi);
            const v16f Dm = __builtin_amdgcn_mfma_f32_32x32x8f16(an, bs, zero16, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r)
              acc_out[sn][sm][r] = fmaf(Dm[r], nv[r], fmaf(acc[sn][sm][r], dv[r], acc_out[sn][sm][r]));
          }
        }
      }
    }
  }
#undef BQMM_FETCH
#undef BQMM_STAGE

  if constexpr (!kDump) {
    const bool full = (m_base + BM <= m) && (n_base + BN <= n) && (ldc % 4u) == 0u;
#pragma unroll
    for (int sm = 0; sm < 2; ++sm) {
      const uint32_t mloc = wm * 64 + sm * 32 + l32;
      const uint32_t mm = m_base + mloc;
      uint16_t *orow = out + (uint64_t)min(mm, m - 1u) * ldc;
      // undo the activation operand's 2^-e (exact: a power of two)
      const float e2 = __builtin_amdgcn_ldexpf(1.0f, q4k_rowexp[mloc] - 23);
#pragma unroll
      for (int sn = 0; sn < 2; ++sn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t nn = n_base + wn * 64 + sn * 32 + 8 * q + 4 * hi;
          v16f v = acc_out[sn][sm];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[4 * q + e] *= e2;
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
  // The stages exceed the 64 KB default dynamic-LDS limit; gfx950 allows 160 KB.
  hipError_t attr_err = ensure_dynamic_lds(reinterpret_cast<const void *>(q4k_mmq_kernel<false>), kLdsBytes);
  if (attr_err == hipSuccess)
    attr_err = ensure_dynamic_lds(reinterpret_cast<const void *>(q4k_mmq_kernel<true>), kLdsBytes);
  if (attr_err != hipSuccess) return attr_err;
  if (dots == nullptr) {
    const dim3 grid((uint32_t)(((uint64_t)n + BN - 1) / BN), (uint32_t)(((uint64_t)m + BM - 1) / BM));
    hipLaunchKernelGGL(q4k_mmq_kernel<false>, grid, dim3(kThreads), kLdsBytes, s,
                       static_cast<const uint8_t *>(act_q8), static_cast<const uint8_t *>(w),
                       static_cast<uint16_t *>(out), nullptr, m, n, k, 0u, 0u, 0u, 0u, 0u, 0u, ldc);
  } else {
    const uint32_t tn0 = n0 / BN, tn1 = (n0 + nt - 1) / BN;
    const uint32_t tm0 = m0 / BM, tm1 = (m0 + mt - 1) / BM;
    const dim3 grid(tn1 - tn0 + 1, tm1 - tm0 + 1);
    hipLaunchKernelGGL(q4k_mmq_kernel<true>, grid, dim3(kThreads), kLdsBytes, s,
                       static_cast<const uint8_t *>(act_q8), static_cast<const uint8_t *>(w),
                       nullptr, dots, m, n, k, m0, mt, n0, nt, tn0, tm0, n);
  }
  return hipGetLastError();
}

}  // namespace bqmm

// Q2_0 GEMV for small verify batches (m = 2..8) on bf16 matrix cores.
//
// [page layers/dense_ffn_decode_batch.rs, fn forward_km_q2:
//  q2_0_gemv_vec_batchm on the bf16 activations, output bf16.]
//
// out[i][r] = sum_k a[i][k] * d[r][g] * (c - 2), fp32 accumulation.
//
// With m activation rows every code feeds m multiply-adds.  On the vector
// ALU that work grows with m (two per v_dot2), so this kernel moves the
// products to v_mfma_f32_16x16x32_bf16 and keeps the VALU for the
// m-independent part: turning codes into bf16 (about 0.75 ops per code).
// The dispatcher uses it only where the per-code ALU work of the vector
// kernel is larger.
//
// Operands of one MFMA (field j of a 128-group, i.e. the 32 k of block j):
//   A = 16 weight rows x 32 k; lane l holds row l % 16 and, with lg = l / 16,
//       the 8 consecutive k = bo .. bo + 7 of field j, bo = 16 (lg & 1) +
//       8 (lg >> 1), i.e. bytes bo .. bo + 7 of the row's group (the four
//       lane groups cover the 32 bytes in a permuted order), code field j,
//       as bf16 2^e_j + c (mantissa OR, exact; e = 7, 5, 3, 2);
//   B = the same 32 k x 16 columns; column j' < m is activation row j',
//       loaded as 8 consecutive bf16 straight from memory (columns >= m
//       repeat row m - 1 and their outputs are dropped);
//   D = 16 x 16 fp32; lane l holds column l % 16, rows 4 (l / 16) .. +3.
// Weight loads take two groups (64 bytes of a row) at once, four consecutive
// lanes on one row's 64 bytes (lane l: row l / 4, 16-byte chunk l % 4), so an
// instruction covers 16 rows x 64 contiguous bytes.  A wave hands each tile's
// load to the MFMA layout through 1 KB of LDS (one 16-byte store and one load
// per lane, conflict-free) and then one v_permlane32_swap per dword splits
// the pair into the two groups' A words.  Against the earlier loads of one
// group per instruction, 8 bytes per lane on 16 rows x 32 bytes (A/B on one
// machine at m = 4 / 6 / 8, identical results between the two new versions):
// the pair loads alone took the down projection [5120, 17408] from 19.1 /
// 20.3 / 22.7 to 16.9 / 18.0 / 20.4 us; with four consecutive lanes per row
// segment (instead of lanes 16 apart) to 14.9 / 15.4 / 17.6 us; the gate
// [17408, 5120] from 14.7 / 15.2 / 15.9 to 12.2 / 12.5 / 13.2 us and the
// fused gate/up from 27.1 / 27.8 / 28.6 to 24.0 / 24.4 / 25.4 us.  Timing-only
// copies with whole 128-byte row segments per instruction (8 rows each) ran
// the gate in 11.1-11.7 us, but the quad-of-groups pipeline they need measured
// slower than the pair one.
// The constant part of the codes is removed by four more MFMAs per group with
// A = -(2^e_j + 2) everywhere: their sum, -sum_k (2^e + 2) a_k for every row,
// is the accumulator the weight MFMAs start from, so each group's result is
// sum_k (c_k - 2) a_k exactly as the four weight MFMAs see it.  It is shared
// by the T row tiles a wave processes.  The group scale is applied once per
// group and output with an fma.
//
// Work split: a wave owns T tiles of 16 rows and a contiguous range of the
// 128-groups; the W waves of a workgroup split k between them and add their
// partial sums through LDS at the end.  The T tiles share each activation
// load (four per group and lane; with two tiles, on the down projection, a
// timing copy that issued half of them ran 13% faster at m = 8, with five no
// faster), so T is as large as the launch allows: the grid must fit the
// compute units in one round (a second, partial round of these
// latency-bound waves nearly doubles the time).  Measured on the FFN shapes
// at m = 8 with the one-group loads: wide single (n = 17408) T = 3 within
// 128 VGPRs, so
// two 8-wave workgroups share a CU and all 363 fit at once (20.4 us, was 25.4
// with T = 2 at 134 VGPRs, one workgroup per CU and 544 of them); narrow
// (n = 5120) T = 2, 160 workgroups (24.7 us, was 31.2 with T = 1); fused
// gate/up T = 3 of each weight (36.7 us, was 46.1 with T = 1).
// Balanced rows: where that grid has more workgroups than the chip has
// compute units, some units run two workgroups and others one, and the units
// with two set the time.  The launch then gives every unit one workgroup of
// rb = ceil(n / CUs) rows (68 for n = 17408 on 256 units) in T = ceil(rb / 16)
// tiles, the last one starting at row rb - 16 so that it overlaps its
// neighbour inside the workgroup (no row is loaded by two workgroups; the
// overlapped rows are stored once).  A/B on one machine, m = 4 / 6 / 8, identical
// outputs (with the one-group loads of that time): gate 17.0 / 17.7 / 19.2 ->
// 14.7 / 15.2 / 15.9 us, fused gate/up
// 29.8 / 30.9 / 32.5 -> 27.1 / 27.8 / 28.6 us.  The narrow down projection
// (160 workgroups, one per unit) gains nothing from it: split into 256
// workgroups of 20 rows it measured 2% slower.  There is no barrier in the
// main loop.  A wave's weight scales are staged once in LDS
// ([group][row], so one 8-byte read gives the four rows of a lane's
// outputs).  Loads run P pairs of groups ahead, unconditionally from clamped
// addresses.
#include "gemv_common.h"

namespace bqmm {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v8bf as_bf8(v4u x) { return __builtin_bit_cast(v8bf, x); }

__device__ __forceinline__ v4f mfma(v4u a, v4u b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(a), as_bf8(b), c, 0, 0, 0);
}

#ifndef BQMM_GEMVX_WIDE_N
#define BQMM_GEMVX_WIDE_N 8192
#endif
constexpr int kStageBatch = 8;  // scale-staging loads per lane per round

template <int M, int T, int W, int P, int NW, int MINW>
__global__ __launch_bounds__(64 * W, MINW) void q2_0_gemv_mfma_kernel(const uint16_t *__restrict__ act,
                                                                const uint8_t *__restrict__ w,
                                                                const uint8_t *__restrict__ w2,
                                                                uint16_t *__restrict__ out,
                                                                uint32_t n, uint32_t k, uint32_t rb) {
  static_assert(M >= 1 && M <= 16, "one MFMA column per activation row");
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  static_assert(NW == 1 || NW == 2, "one weight, or gate and up");
  constexpr uint32_t kRows = 16 * T;
  constexpr int TT = NW * T;  // tile slots: T of each weight (same rows)
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint32_t lr = lane & 15u, lg = lane >> 4;
  const uint32_t G = k >> 7;
  const uint32_t gmax = (G + W - 1) / W;  // groups of the widest wave
  const uint32_t gb = wave * G / W, ng = (wave + 1) * G / W - gb;  // >= 1 since G >= W
  // rb rows per workgroup (16 <= rb <= 16 T); tile t starts at row min(16 t, rb - 16)
  const uint32_t row0 = blockIdx.x * rb;

  // Weight loads: lane l takes row l / 4 of each tile and 16-byte chunk l % 4
  // of a pair of groups (four consecutive lanes on 64 contiguous bytes of a
  // row; with a single group per row, chunk l % 2 of it).  Rows past n read
  // row n - 1 and are not stored; slots T .. 2T-1 are the up rows.
  const uint8_t *wp[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const uint32_t row = min(row0 + min(16u * (t % T), rb - 16u) + (lane >> 2), n - 1u);
    wp[t] = (t < T ? w : w2) + (uint64_t)row * (k >> 2) + 16u * (G >= 2 ? (lane & 3u) : (lane & 1u));
  }
  // a wave's 1 KB through which each tile's pair load is handed to the lanes
  // of the MFMA layout: lane s stores at slot s ^ ((s >> 4) & 3) and lane
  // (lr, lg) loads the slot of lane 4 lr + lg (both conflict-free)
  v4u *tbuf = reinterpret_cast<v4u *>(reinterpret_cast<uint8_t *>(smem) +
                                          ((2u * W * NW * kRows * gmax + 15u) & ~15u)) + 64u * wave;
  const uint32_t wslot = lane ^ ((lane >> 4) & 3u);
  const uint32_t src = 4u * lr + lg, rslot = src ^ ((src >> 4) & 3u);
  // activation offset of the lane's eight k in each field: lane group lg
  // supplies group bytes 16 (lg & 1) + 8 (lg >> 1) .. +7 (see the pair swap)
  const uint32_t bo = 16u * (lg & 1u) + 8u * (lg >> 1);
  const uint16_t *ap = act + (uint64_t)min(lr, (uint32_t)M - 1u) * k + bo;
  const uint32_t npair = (ng + 1u) >> 1;

  uint4 cq[P][TT];
  uint4 aq[P][8];
  // slot <- pair pi: groups 2 pi, 2 pi + 1 of the wave (clamped to its last);
  // the weight load covers the pair of groups starting at ps = min(gA, G - 2)
#define BQMM_LOADX(slot, pi)                                                        \
  do {                                                                              \
    const uint32_t gA_ = gb + min(2u * (uint32_t)(pi), ng - 1u);                    \
    const uint32_t gB_ = gb + min(2u * (uint32_t)(pi) + 1u, ng - 1u);               \
    const uint32_t ps_ = G >= 2 ? min(gA_, G - 2u) : 0u;                            \
    _Pragma("unroll") for (int t = 0; t < TT; ++t)                                  \
      cq[slot][t] = *reinterpret_cast<const uint4 *>(wp[t] + 32u * ps_);            \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                   \
      aq[slot][j] = *reinterpret_cast<const uint4 *>(ap + 128u * gA_ + 32u * j);    \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                   \
      aq[slot][4 + j] = *reinterpret_cast<const uint4 *>(ap + 128u * gB_ + 32u * j); \
  } while (0)

  // Stage this wave's scales in LDS: [weight][group][row] fp16.  A round
  // issues kStageBatch loads per lane before storing any, and the first round
  // goes out before the weight prefetch: vector-memory counters retire in
  // order, so stores placed after the prefetch would wait for its HBM loads,
  // and a load-store loop would pay one memory latency per iteration.
  // Entries are numbered group-major (consecutive lanes take consecutive rows,
  // so the LDS writes are contiguous and the row index is a division by a
  // constant).
  uint16_t *sc = reinterpret_cast<uint16_t *>(smem) + wave * (NW * kRows * gmax);
  const uint32_t per_w = kRows * ng, nst = NW * per_w;
  auto stage_round = [&](uint32_t base) {
    uint32_t v[kStageBatch], dst[kStageBatch];
#pragma unroll
    for (int b = 0; b < kStageBatch; ++b) {
      const uint32_t i = min(base + lane + 64u * b, nst - 1u);
      const uint32_t wv = i >= per_w ? 1u : 0u, rem = i - wv * per_w;
      const uint32_t gi = rem / kRows, r = rem - gi * kRows;
      const uint16_t *scales = reinterpret_cast<const uint16_t *>((wv == 0 ? w : w2) + (uint64_t)n * k / 4u);
      v[b] = scales[(uint64_t)min(row0 + min(r & ~15u, rb - 16u) + (r & 15u), n - 1u) * G + gb + gi];
      dst[b] = (wv * gmax + gi) * kRows + r;
    }
#pragma unroll
    for (int b = 0; b < kStageBatch; ++b)
      if (base + lane + 64u * b < nst) sc[dst[b]] = (uint16_t)v[b];
  };
  stage_round(0);

#pragma unroll
  for (int p = 0; p < P; ++p) BQMM_LOADX(p, p);

  for (uint32_t base = 64u * kStageBatch; base < nst; base += 64u * kStageBatch) stage_round(base);

  const uint32_t M0 = vconst(0x00030003u), M1 = vconst(0x000C000Cu), M2 = vconst(0x00300030u),
                 M3 = vconst(0x00600060u);
  const uint32_t G0 = vconst(0x43004300u), G1 = vconst(0x42004200u), G2 = vconst(0x41004100u),
                 G3 = vconst(0x40804080u);
  // -(2^e_j + 2) = -130, -34, -10, -6 in bf16, eight per lane
  const v4u NK[4] = {v4u{0xC302C302u, 0xC302C302u, 0xC302C302u, 0xC302C302u},
                     v4u{0xC208C208u, 0xC208C208u, 0xC208C208u, 0xC208C208u},
                     v4u{0xC120C120u, 0xC120C120u, 0xC120C120u, 0xC120C120u},
                     v4u{0xC0C0C0C0u, 0xC0C0C0C0u, 0xC0C0C0C0u, 0xC0C0C0C0u}};

  v4f acc_out[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc_out[t] = v4f{0.f, 0.f, 0.f, 0.f};

  // bytes of a code word reordered to (b0, b2, b1, b3): b0/b1 then sit in the
  // low bytes of the two halves (fields at bits 2j, 16 + 2j), b2/b3 after >> 8
// one group: its A words (x0w, x1w: the lane's eight code bytes), its
// activation operands aq[slot][ab .. ab + 3] and wave-relative index gi
#define BQMM_GROUP(x0w, x1w, slot, ab, t, gi)                                       \
  do {                                                                              \
    const uint16_t *srow_ = sc + (((t) / T) * gmax + (uint32_t)(gi)) * kRows + 4u * lg; \
    const uint32_t x0_ = __builtin_amdgcn_perm((x0w), (x0w), 0x03010200u);          \
    const uint32_t x1_ = __builtin_amdgcn_perm((x1w), (x1w), 0x03010200u);          \
    const uint32_t y0_ = x0_ >> 8, y1_ = x1_ >> 8;                                  \
    const v4u a0_ = {and_or(x0_, M0, G0), and_or(y0_, M0, G0), and_or(x1_, M0, G0), and_or(y1_, M0, G0)}; \
    const v4u a1_ = {and_or(x0_, M1, G1), and_or(y0_, M1, G1), and_or(x1_, M1, G1), and_or(y1_, M1, G1)}; \
    const v4u a2_ = {and_or(x0_, M2, G2), and_or(y0_, M2, G2), and_or(x1_, M2, G2), and_or(y1_, M2, G2)}; \
    const v4u a3_ = {and_or(x0_ >> 1, M3, G3), and_or(y0_ >> 1, M3, G3),          \
                     and_or(x1_ >> 1, M3, G3), and_or(y1_ >> 1, M3, G3)};         \
    v4f s_ = mfma(a0_, v4u{aq[slot][ab].x, aq[slot][ab].y, aq[slot][ab].z, aq[slot][ab].w}, nb_); \
    s_ = mfma(a1_, v4u{aq[slot][ab + 1].x, aq[slot][ab + 1].y, aq[slot][ab + 1].z, aq[slot][ab + 1].w}, s_); \
    s_ = mfma(a2_, v4u{aq[slot][ab + 2].x, aq[slot][ab + 2].y, aq[slot][ab + 2].z, aq[slot][ab + 2].w}, s_); \
    s_ = mfma(a3_, v4u{aq[slot][ab + 3].x, aq[slot][ab + 3].y, aq[slot][ab + 3].z, aq[slot][ab + 3].w}, s_); \
    const uint2 dv_ = *reinterpret_cast<const uint2 *>(srow_ + 16u * ((t) % T));    \
    acc_out[t][0] = fmaf(f16_bits_to_f32(dv_.x & 0xFFFFu), s_[0], acc_out[t][0]);   \
    acc_out[t][1] = fmaf(f16_bits_to_f32(dv_.x >> 16), s_[1], acc_out[t][1]);       \
    acc_out[t][2] = fmaf(f16_bits_to_f32(dv_.y & 0xFFFFu), s_[2], acc_out[t][2]);   \
    acc_out[t][3] = fmaf(f16_bits_to_f32(dv_.y >> 16), s_[3], acc_out[t][3]);       \
  } while (0)
#define BQMM_BIAS(slot, ab)                                                         \
  do {                                                                              \
    nb_ = v4f{0.f, 0.f, 0.f, 0.f};                                                  \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                 \
      const v4u b_ = {aq[slot][ab + j].x, aq[slot][ab + j].y, aq[slot][ab + j].z, aq[slot][ab + j].w}; \
      nb_ = mfma(NK[j], b_, nb_);                                                   \
    }                                                                               \
  } while (0)
  // A pair of groups: lane (lr, lg) holds bytes 16 lg .. +15 of the pair's
  // 64 bytes of row lr.  One v_permlane32_swap per dword (lanes 32..63 of the
  // first operand trade places with lanes 0..31 of the second) leaves the
  // first group's bytes 16 (lg & 1) + 8 (lg >> 1) .. +7 in the first result
  // and the second group's in the second.
#define BQMM_COMPUTEX(slot, pi)                                                     \
  do {                                                                              \
    const uint32_t gi_ = 2u * (uint32_t)(pi);                                       \
    const uint32_t gA_ = gb + gi_;                                                  \
    const uint32_t pos_ = G >= 2 ? gA_ - min(gA_, G - 2u) : 0u;                    \
    v4u tv_[TT];                                                                    \
    _Pragma("unroll") for (int t = 0; t < TT; ++t) {                                \
      tbuf[wslot] = v4u{cq[slot][t].x, cq[slot][t].y, cq[slot][t].z, cq[slot][t].w}; \
      __builtin_amdgcn_wave_barrier();                                              \
      tv_[t] = tbuf[rslot];                                                         \
      __builtin_amdgcn_wave_barrier();                                              \
    }                                                                               \
    v4f nb_;                                                                        \
    if (gi_ + 1u < ng) {                                                            \
      BQMM_BIAS(slot, 0);                                                           \
      _Pragma("unroll") for (int t = 0; t < TT; ++t) {                              \
        const v4u v_ = tv_[t];                                                      \
        const auto sx_ = __builtin_amdgcn_permlane32_swap(v_.x, v_.z, false, false); \
        const auto sy_ = __builtin_amdgcn_permlane32_swap(v_.y, v_.w, false, false); \
        BQMM_GROUP(sx_[0], sy_[0], slot, 0, t, gi_);                                \
      }                                                                             \
      BQMM_BIAS(slot, 4);                                                           \
      _Pragma("unroll") for (int t = 0; t < TT; ++t) {                              \
        const v4u v_ = tv_[t];                                                      \
        const auto sx_ = __builtin_amdgcn_permlane32_swap(v_.x, v_.z, false, false); \
        const auto sy_ = __builtin_amdgcn_permlane32_swap(v_.y, v_.w, false, false); \
        BQMM_GROUP(sx_[1], sy_[1], slot, 4, t, gi_ + 1u);                           \
      }                                                                             \
    } else {                                                                        \
      BQMM_BIAS(slot, 0);                                                           \
      _Pragma("unroll") for (int t = 0; t < TT; ++t) {                              \
        const v4u v_ = tv_[t];                                                      \
        const auto sx_ = __builtin_amdgcn_permlane32_swap(v_.x, v_.z, false, false); \
        const auto sy_ = __builtin_amdgcn_permlane32_swap(v_.y, v_.w, false, false); \
        BQMM_GROUP(pos_ ? sx_[1] : sx_[0], pos_ ? sy_[1] : sy_[0], slot, 0, t, gi_); \
      }                                                                             \
    }                                                                               \
  } while (0)

  uint32_t pi0 = 0;
  for (; pi0 + P <= npair; pi0 += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      BQMM_COMPUTEX(u, pi0 + u);
      BQMM_LOADX(u, pi0 + u + P);
    }
  }
  // the last npair - pi0 < P pairs are already loaded
#pragma unroll
  for (int u = 0; u < P - 1; ++u)
    if (pi0 + u < npair) BQMM_COMPUTEX(u, pi0 + u);
#undef BQMM_LOADX
#undef BQMM_COMPUTEX
#undef BQMM_GROUP
#undef BQMM_BIAS

  // add the W waves' partial sums: red[wave][t][i][lane]
  __syncthreads();  // every wave is done with its scales (the same LDS)
  float *red = reinterpret_cast<float *>(smem);
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((wave * TT + t) * 4 + i) * 64 + lane] = acc_out[t][i];
  __syncthreads();
  for (uint32_t o = tid; o < kRows * M; o += 64u * W) {
    const uint32_t col = o / kRows, r = o - col * kRows;
    const uint32_t t = r >> 4, rr = r & 15u;
    const uint32_t src = ((t * 4 + (rr & 3u)) * 64) + (rr >> 2) * 16 + col;
    float s = 0.0f;
#pragma unroll
    for (int v = 0; v < W; ++v) s += red[v * TT * 256 + src];
    uint32_t h = f32_to_bf16_rne(s);
    if (NW == 2) {
      // the up row's sum, then silu(gate) * up on both values rounded to bf16
      float su = 0.0f;
#pragma unroll
      for (int v = 0; v < W; ++v) su += red[v * TT * 256 + T * 256 + src];
      h = f32_to_bf16_rne(silu_mul_f32(bf16_to_f32(h), bf16_to_f32(f32_to_bf16_rne(su))));
    }
    // a row of the last tile that the tile before it covers is stored by that tile
    const uint32_t lr0 = min(16u * t, rb - 16u) + rr;
    if (lr0 >= 16u * t && lr0 < rb && row0 + lr0 < n) out[(uint64_t)col * n + row0 + lr0] = (uint16_t)h;
  }
}

// Dynamic LDS of a launch with W waves of T tiles: the staged weight scales
// of a wave's groups and each wave's 1 KB for the weight loads, or the
// partial sums of the final reduction.
inline size_t lds_bytes(int W, int T, int NW, uint32_t k) {
  const uint32_t G = k >> 7;
  const uint32_t gmax = (G + W - 1) / W;
  const size_t sc_bytes = (((size_t)W * NW * 16 * T * gmax * 2 + 15) & ~(size_t)15) + (size_t)W * 1024;
  const size_t red_bytes = (size_t)W * NW * T * 4 * 64 * 4;
  return sc_bytes > red_bytes ? sc_bytes : red_bytes;
}

template <int M, int W, int T, int NW, int MINW, int P>
hipError_t launch_w(const void *act, const void *w, const void *w2, void *out, uint32_t n, uint32_t k,
                    hipStream_t s) {
  const size_t lds = lds_bytes(W, T, NW, k);
  if (lds > 65536) return hipErrorInvalidValue;  // the dispatcher checks q2_0_gemv_mfma_fits first
  const uint32_t blocks = (n + 16 * T - 1) / (16 * T);
  hipLaunchKernelGGL((q2_0_gemv_mfma_kernel<M, T, W, P, NW, MINW>), dim3(blocks), dim3(64 * W), lds, s,
                     static_cast<const uint16_t *>(act), static_cast<const uint8_t *>(w),
                     static_cast<const uint8_t *>(w2), static_cast<uint16_t *>(out), n, k, 16u * T);
  return hipGetLastError();
}

// The balanced launch: one workgroup of rb rows per compute unit.  Its dynamic
// LDS is raised to at least kBalancedMinLds, more than half a unit's 160 KB,
// so that no unit takes two of them.
constexpr size_t kBalancedMinLds = 81 * 1024;
constexpr size_t kMaxLds = 160 * 1024;
template <int M, int T, int NW, int P>
hipError_t launch_balanced(const void *act, const void *w, const void *w2, void *out, uint32_t n, uint32_t k,
                           uint32_t rb, hipStream_t s) {
  constexpr int W = 8;
  size_t lds = lds_bytes(W, T, NW, k);
  if (lds > kMaxLds) return hipErrorInvalidValue;  // checked by balanced_rows first
  if (lds < kBalancedMinLds) lds = kBalancedMinLds;
  const hipError_t e =
      ensure_dynamic_lds(reinterpret_cast<const void *>(q2_0_gemv_mfma_kernel<M, T, W, P, NW, 1>), (int)lds);
  if (e != hipSuccess) return e;
  const uint32_t blocks = (n + rb - 1) / rb;
  hipLaunchKernelGGL((q2_0_gemv_mfma_kernel<M, T, W, P, NW, 1>), dim3(blocks), dim3(64 * W), lds, s,
                     static_cast<const uint16_t *>(act), static_cast<const uint8_t *>(w),
                     static_cast<const uint8_t *>(w2), static_cast<uint16_t *>(out), n, k, rb);
  return hipGetLastError();
}

// Eight waves split k when it has at least eight groups (W <= G is required).
// The tiles per wave and the register bound (minimum waves per SIMD) are set
// per case below.  The fused gate/up kernel takes T tiles of each weight (the
// same rows) and the same k split, so per-row sums are identical to the
// single kernel's.
#ifndef BQMM_GEMVX_T_WIDE
#define BQMM_GEMVX_T_WIDE 3
#endif
#ifndef BQMM_GEMVX_T_NARROW
#define BQMM_GEMVX_T_NARROW 2
#endif
#ifndef BQMM_GEMVX_T_FUSED
#define BQMM_GEMVX_T_FUSED 3
#endif
// (The wide launch reaches the plain grid only where it fits the compute units
// once, one workgroup each, so it no longer needs the 128-VGPR bound that let
// two of them share a unit.)
#ifndef BQMM_GEMVX_MINW_WIDE
#define BQMM_GEMVX_MINW_WIDE 2
#endif
#ifndef BQMM_GEMVX_MINW_NARROW
#define BQMM_GEMVX_MINW_NARROW 2
#endif
#ifndef BQMM_GEMVX_MINW_FUSED
#define BQMM_GEMVX_MINW_FUSED 2
#endif
// Pairs of groups whose loads are in flight per wave (P): one, except on the
// narrow launch (two tiles per wave), where two pairs measured 1-4% faster at
// m = 3, 4, 8 on the down projection; on the five-tile gate two pairs were 8%
// slower and the fused kernel spills with them.  (With one group per load, two
// groups in flight had been the best choice for the wide kernel.)  The depth
// does not change the order of any sum.
constexpr int kPairsInFlight = 1;
constexpr int kPairsInFlightNarrow = 2;
// The launch shape launch_m picks for (n, k): waves W and tiles per wave T.
inline void launch_shape(uint32_t n, uint32_t k, int NW, int &W, int &T) {
  if ((k >> 7) >= 8) {
    W = 8;
    T = NW == 2 ? BQMM_GEMVX_T_FUSED : (n >= BQMM_GEMVX_WIDE_N ? BQMM_GEMVX_T_WIDE : BQMM_GEMVX_T_NARROW);
  } else {
    W = 1;
    T = 2;
  }
}

// Rows per workgroup of the balanced launch for (n, k), or 0 where the plain
// grid (T tiles per workgroup) fits the compute units in one workgroup each,
// or the balanced tile count is outside 4..6 (4..5 for two weights: six tiles
// of each spill registers), or its LDS does not fit.
inline uint32_t balanced_rows(uint32_t n, uint32_t k, int NW, int T) {
  int cus = 0;
  if (device_cu_count(&cus) != hipSuccess || cus <= 0) return 0;
  const uint32_t ncu = (uint32_t)cus;
  if ((n + 16u * T - 1) / (16u * T) <= ncu) return 0;
  const uint32_t rb = (n + ncu - 1) / ncu, tb = (rb + 15) / 16;
  if (tb < 4 || tb > (NW == 2 ? 5u : 6u) || lds_bytes(8, (int)tb, NW, k) > kMaxLds) return 0;
  return rb;
}

template <int M, int NW>
hipError_t launch_m(const void *act, const void *w, const void *w2, void *out, uint32_t n, uint32_t k,
                    hipStream_t s) {
  const uint32_t G = k >> 7;
  if (G >= 8) {
    const int Tp = NW == 2 ? BQMM_GEMVX_T_FUSED : (n >= BQMM_GEMVX_WIDE_N ? BQMM_GEMVX_T_WIDE : BQMM_GEMVX_T_NARROW);
    const uint32_t rb = balanced_rows(n, k, NW, Tp);
    if (rb != 0) {
      constexpr int P = kPairsInFlight;
      switch ((rb + 15) / 16) {
        case 4: return launch_balanced<M, 4, NW, P>(act, w, w2, out, n, k, rb, s);
        case 5: return launch_balanced<M, 5, NW, P>(act, w, w2, out, n, k, rb, s);
        default:
          if constexpr (NW == 1) return launch_balanced<M, 6, NW, P>(act, w, w2, out, n, k, rb, s);
          else return hipErrorInvalidValue;  // balanced_rows allows at most five tiles here
      }
    }
    if constexpr (NW == 2) {
      return launch_w<M, 8, BQMM_GEMVX_T_FUSED, NW, BQMM_GEMVX_MINW_FUSED, kPairsInFlight>(act, w, w2, out, n, k,
                                                                                          s);
    } else {
      if (n >= BQMM_GEMVX_WIDE_N)
        return launch_w<M, 8, BQMM_GEMVX_T_WIDE, NW, BQMM_GEMVX_MINW_WIDE, kPairsInFlight>(act, w, w2, out, n, k,
                                                                                        s);
      return launch_w<M, 8, BQMM_GEMVX_T_NARROW, NW, BQMM_GEMVX_MINW_NARROW, kPairsInFlightNarrow>(act, w, w2, out,
                                                                                                  n, k, s);
    }
  }
  return launch_w<M, 1, 2, NW, 1, kPairsInFlight>(act, w, w2, out, n, k, s);
}


// m below the dispatch threshold never reaches these entry points; those
// sizes are not instantiated.
template <int NW>
hipError_t launch_any_m(const void *act, const void *w, const void *w2, void *out, uint32_t m, uint32_t n,
                        uint32_t k, hipStream_t s) {
  if (m < (uint32_t)BQMM_GEMV_MIN_M_MFMA) return hipErrorInvalidValue;
  switch (m) {
#if BQMM_GEMV_MIN_M_MFMA <= 2
    case 2: return launch_m<2, NW>(act, w, w2, out, n, k, s);
#endif
#if BQMM_GEMV_MIN_M_MFMA <= 3
    case 3: return launch_m<3, NW>(act, w, w2, out, n, k, s);
#endif
#if BQMM_GEMV_MIN_M_MFMA <= 4
    case 4: return launch_m<4, NW>(act, w, w2, out, n, k, s);
#endif
#if BQMM_GEMV_MIN_M_MFMA <= 5
    case 5: return launch_m<5, NW>(act, w, w2, out, n, k, s);
#endif
    case 6: return launch_m<6, NW>(act, w, w2, out, n, k, s);
    case 7: return launch_m<7, NW>(act, w, w2, out, n, k, s);
    case 8: return launch_m<8, NW>(act, w, w2, out, n, k, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool q2_0_gemv_mfma_fits(uint32_t n, uint32_t k, int nw) {
  int W = 1, T = 1;
  launch_shape(n, k, nw, W, T);
  return lds_bytes(W, T, nw, k) <= 65536;
}

hipError_t launch_q2_0_gemv_mfma(const void *act, const void *w, void *out, uint32_t m, uint32_t n,
                                 uint32_t k, hipStream_t s) {
  return launch_any_m<1>(act, w, nullptr, out, m, n, k, s);
}

hipError_t launch_q2_0_gemv_mfma_gate_up(const void *act, const void *w_gate, const void *w_up,
                                         void *out, uint32_t m, uint32_t n, uint32_t k,
                                         hipStream_t s) {
  return launch_any_m<2>(act, w_gate, w_up, out, m, n, k, s);
}

}  // namespace bqmm

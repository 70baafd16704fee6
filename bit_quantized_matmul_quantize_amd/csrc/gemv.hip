// Q2_0 GEMV for decode (m = 1) and small verify batches (m = 2..8).
//
// [page layers/qwen3_ssm/init.rs, kernel q2_0_gemv_vec; page
//  layers/dense_ffn_decode_batch.rs, fn forward_km_q2: q2_0_gemv_vec_batchm on
//  the bf16 activations, output bf16.]
//
// out[i][r] = sum_k a[i][k] * d[r][g] * (c - 2), accumulated in fp32.
// Bandwidth kernels: the packed weight (2.125 bits per weight) is streamed
// once with 16-byte loads, row sums are wavefront reductions, no matrix cores.
//
// Shared arithmetic.  A 16-byte chunk c = 2g + h of a weight row holds 64
// codes: field j (bits 2j..2j+1) of byte t is the code of
// k = 128g + 32j + 16h + t.  Codes become bf16 without a conversion: OR-ing
// the masked field into the mantissa of bf16 2^e gives exactly 2^e + c, with
// e = 7, 5, 3 for j = 0..2 (field at mantissa bits 0, 2, 4) and e = 2 for
// j = 3 (field shifted down one bit to mantissa bits 5..6).  One v_and_or_b32
// builds two such values: bytes 0 and 2 of a 32-bit word land in the low and
// high halves, bytes 1 and 3 after a shift by 8.  The activations are stored
// permuted into the matching pairs (t, t+2), (t+1, t+3), so one
// v_dot2_f32_bf16 adds (2^e + c_t) a_t + (2^e + c_t') a_t'.  Per field the
// partial bias sum_t (2^e + 2) a_t is subtracted once per chunk, leaving
// sum_t (c_t - 2) a_t; then the group scale is applied with one fma.
// Activations are used as given (zeros stay exact zeros).
#include "gemv_common.h"

namespace bqmm {
namespace {

constexpr int kThreads = 256;

// bf16 2^e for the four fields, in both halves
constexpr uint32_t kMagic[4] = {0x43004300u, 0x42004200u, 0x41004100u, 0x40804080u};

struct CodeConsts {
  uint32_t m0, m1, m2, m3, g0, g1, g2, g3;
};

__device__ __forceinline__ CodeConsts code_consts() {
  return {vconst(0x00030003u), vconst(0x000C000Cu), vconst(0x00300030u), vconst(0x00600060u),
          vconst(kMagic[0]),   vconst(kMagic[1]),   vconst(kMagic[2]),   vconst(kMagic[3])};
}

// The eight bf16 pairs of one 32-bit code word, in the order
// (field 0: bytes 0/2, bytes 1/3), (field 1: ...), (field 2: ...), (field 3: ...).
__device__ __forceinline__ void word_pairs(uint32_t x, const CodeConsts &K, uint32_t p[8]) {
  const uint32_t x8 = x >> 8, x1 = x >> 1, x9 = x >> 9;
  p[0] = and_or(x, K.m0, K.g0);
  p[1] = and_or(x8, K.m0, K.g0);
  p[2] = and_or(x, K.m1, K.g1);
  p[3] = and_or(x8, K.m1, K.g1);
  p[4] = and_or(x, K.m2, K.g2);
  p[5] = and_or(x8, K.m2, K.g2);
  p[6] = and_or(x1, K.m3, K.g3);
  p[7] = and_or(x9, K.m3, K.g3);
}

// bf16 pair of 2^e_j + 2 for a field index j that is not a compile-time
// constant (e = 7, 5, 3, 2): exponent 127 + e, one mantissa bit at 8 - e.
// Integer arithmetic rather than a table or a select chain, which the compiler
// turns into divergent branches.
__device__ __forceinline__ uint32_t bias_weight(uint32_t j) {
  const uint32_t e = 7u - 2u * j + ((j >> 1) & j & 1u);
  const uint32_t b = ((127u + e) << 7) | (1u << (8u - e));
  return b | (b << 16);
}

// sum_t (2^e_j + 2) a_t over 16 values
__device__ __forceinline__ float field_bias(const uint32_t D[8], uint32_t bw) {
  float b = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) b = dot2(D[i], bw, b);
  return b;
}

// ---- m = 1 decode kernel ---------------------------------------------------
//
// Each lane keeps one fixed chunk position c of the weight rows and serves
// kRowsPerLane rows; a half-wave (32 lanes) covers 32 consecutive chunks of a
// row per slice.  The whole activation vector is prepared once per workgroup
// in LDS (pairs field-major: dword 8j + 2i + b of a chunk, then the four
// partial biases), one lane per (chunk, field).  The weight loads of the first
// slice are issued right after the first prep item's activation loads and
// stay in flight during the prep.  Per row and chunk: 12 shifts,
// 32 v_and_or_b32, 32 v_dot2 and one fma for 64 codes.

#ifndef BQMM_GEMV_ROWS
#define BQMM_GEMV_ROWS 3
#endif
constexpr int kRowsPerLane = BQMM_GEMV_ROWS;
constexpr int kChunkStride = 36;  // dwords per chunk in LDS: 32 pairs, 4 partial biases
constexpr uint32_t kMaxK1 = 32768;
constexpr uint32_t kMinMMfma = BQMM_GEMV_MIN_M_MFMA;

__global__ __launch_bounds__(kThreads) void q2_0_gemv1_kernel(const uint16_t *__restrict__ act,
                                                              const uint8_t *__restrict__ w,
                                                              uint16_t *__restrict__ out, uint32_t n,
                                                              uint32_t k) {
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  const uint32_t C = k >> 6;  // chunks per row
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint32_t s = lane & 31u, half = lane >> 5;
  const uint32_t row_base = blockIdx.x * (8 * kRowsPerLane) + (wave * 2 + half) * kRowsPerLane;
  const uint16_t *scales = reinterpret_cast<const uint16_t *>(w + (uint64_t)n * k / 4u);
  const uint32_t G = k >> 7;
  const uint32_t nslices = (C + 31u) >> 5;

  // Loads are unconditional, from clamped addresses: a row past n computes on
  // row n-1 and is not stored, a chunk past C is loaded but skipped.  With
  // a branch around each load the compiler must drain the load before the
  // other branch writes the register, which serializes the loads.
  uint4 wq[kRowsPerLane];
  uint32_t sc[kRowsPerLane];
  auto load_slice = [&](uint32_t cs) {
    const uint32_t c = min(s + 32u * cs, C - 1u);
#pragma unroll
    for (int r = 0; r < kRowsPerLane; ++r) {
      const uint32_t row = min(row_base + r, n - 1u);
      wq[r] = *reinterpret_cast<const uint4 *>(w + (uint64_t)row * (k >> 2) + 16u * c);
      sc[r] = scales[(uint64_t)row * G + (c >> 1)];
    }
  };

  // Activation prep: one lane per (chunk, field).  The activation loads of the
  // first item are issued before the weight loads: vector-memory counters
  // retire in issue order, so the prep then waits only for the activations
  // (L2-resident) and not for the weights (HBM).
  auto act_src = [&](uint32_t item) {
    const uint32_t c = item >> 2, j = item & 3u;
    return act + 128u * (c >> 1) + 32u * j + 16u * (c & 1u);
  };
  auto prep = [&](uint32_t item, uint4 av0, uint4 av1) {
    const uint32_t c = item >> 2, j = item & 3u;
    const uint32_t D[8] = {av0.x, av0.y, av0.z, av0.w, av1.x, av1.y, av1.z, av1.w};
    uint32_t p[8];
    act_pairs(D, p);
    const float b = field_bias(D, bias_weight(j));
    uint32_t *dst = smem + c * kChunkStride;
    *reinterpret_cast<uint4 *>(dst + 8 * j) = make_uint4(p[0], p[1], p[2], p[3]);
    *reinterpret_cast<uint4 *>(dst + 8 * j + 4) = make_uint4(p[4], p[5], p[6], p[7]);
    dst[32 + j] = __float_as_uint(b);
  };
  const uint32_t items = 4u * C;
  {
    // first item, peeled so that its loads stay ahead of the weight loads
    const uint32_t first = min(tid, items - 1u);
    const uint4 av0 = *reinterpret_cast<const uint4 *>(act_src(first));
    const uint4 av1 = *reinterpret_cast<const uint4 *>(act_src(first) + 8);
    load_slice(0);
    // Lanes past the last item redo that item (same values to the same LDS
    // words): no branch, so the compiler keeps the loads above in place.
    prep(first, av0, av1);
  }
  for (uint32_t item = tid + kThreads; item < items; item += kThreads)
    prep(item, *reinterpret_cast<const uint4 *>(act_src(item)),
         *reinterpret_cast<const uint4 *>(act_src(item) + 8));
  __syncthreads();

  const CodeConsts K = code_consts();
  float acc_out[kRowsPerLane];
#pragma unroll
  for (int r = 0; r < kRowsPerLane; ++r) acc_out[r] = 0.0f;

  for (uint32_t cs = 0; cs < nslices; ++cs) {
    if (cs > 0) load_slice(cs);
    const uint32_t c = s + 32u * cs;
    if (c < C) {
      const uint32_t *src = smem + c * kChunkStride;
      uint32_t P[32];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint4 t = *reinterpret_cast<const uint4 *>(src + 4 * q);
        P[4 * q] = t.x; P[4 * q + 1] = t.y; P[4 * q + 2] = t.z; P[4 * q + 3] = t.w;
      }
      const uint4 bq = *reinterpret_cast<const uint4 *>(src + 32);
      const float bias = (__uint_as_float(bq.x) + __uint_as_float(bq.y)) +
                         (__uint_as_float(bq.z) + __uint_as_float(bq.w));
#pragma unroll
      for (int r = 0; r < kRowsPerLane; ++r) {
        const uint32_t words[4] = {wq[r].x, wq[r].y, wq[r].z, wq[r].w};
        float acc = -bias;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t wp[8];
          word_pairs(words[i], K, wp);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc = dot2(wp[2 * j], P[8 * j + 2 * i], acc);
            acc = dot2(wp[2 * j + 1], P[8 * j + 2 * i + 1], acc);
          }
        }
        acc_out[r] = fmaf(f16_bits_to_f32(sc[r]), acc, acc_out[r]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kRowsPerLane; ++r) acc_out[r] = half_wave_sum(acc_out[r]);
  if (s == 31u) {
#pragma unroll
    for (int r = 0; r < kRowsPerLane; ++r) {
      const uint32_t row = row_base + r;
      if (row < n) out[row] = (uint16_t)f32_to_bf16_rne(acc_out[r]);
    }
  }
}

// ---- batched kernel, m = 1..8 ---------------------------------------------
//
// Used for the verify batches, and for m = 1 when k is beyond the decode
// kernel's whole-vector LDS staging.  A group of L lanes serves R weight rows;
// lane li of the group takes chunk li of every slice of L chunks.  The
// workgroup (256 / L groups, 256 R / L rows) walks k slice by slice: the
// activation slice of all M rows is prepared into LDS once per workgroup and
// read by every group, so the prep is amortized over the workgroup's rows and
// each activation pair read from LDS feeds R rows.
//
// LDS per chunk and activation row (kRowDw dwords): 32 pairs word-major
// (dword 8i + 2j + b for word i, field j, byte pair b), then the four partial
// biases; chunks are padded so that the 16 chunks read by one instruction hit
// distinct bank quads.  Two LDS buffers and D register slots of weights:
// iteration s computes slice s, prepares slice s+1 from activations loaded in
// the previous iteration, loads the activations of slice s+2 and then the
// weights of slice s+D, and ends with the only barrier.  Issuing activation
// loads ahead of weight loads matters because vector-memory counters retire
// in order: the prep of slice s+1 then never waits for HBM.
//
// Chunks past k (a ragged last slice) get zero activations and zero biases,
// so their (clamped, valid) weight loads add exactly 0.

constexpr int kRowDw = 36;

__host__ __device__ constexpr int gemvm_chunk_dwords(int M) {
  return ((kRowDw * M / 4) % 2 == 1) ? kRowDw * M : kRowDw * M + 4;
}

template <int M, int R, int L, int D, int NW>
__global__ __launch_bounds__(kThreads) void q2_0_gemvm_kernel(const uint16_t *__restrict__ act,
                                                              const uint8_t *__restrict__ w,
                                                              const uint8_t *__restrict__ w2,
                                                              uint16_t *__restrict__ out, uint32_t n,
                                                              uint32_t k) {
  static_assert(L == 16 || L == 32, "lane group of 16 or 32");
  static_assert(D == 2 || D == 3, "the load-free tail covers at most two slices");
  static_assert(NW == 1 || NW == 2, "one weight, or gate and up");
  constexpr int RR = NW * R;  // weight rows per lane: R rows of each weight
  constexpr int CS = gemvm_chunk_dwords(M);
  constexpr int kGroups = kThreads / L;
  constexpr int kItems = 4 * L * M;  // prep items per slice: (chunk, field, activation row)
  constexpr int kPrep = (kItems + kThreads - 1) / kThreads;
  static_assert(kItems % 64 == 0, "prep items fill whole waves");
  constexpr int kBuf = L * CS;
  __shared__ __attribute__((aligned(16))) uint32_t lds[2 * kBuf];

  const uint32_t C = k >> 6, G = k >> 7;
  const uint32_t tid = threadIdx.x, li = tid % L, grp = tid / L;
  const uint32_t row_base = (blockIdx.x * kGroups + grp) * R;
  const uint32_t ns = (C + L - 1) / L;

  // rows past n compute on row n-1 and are not stored; with two weights, lane
  // rows R .. 2R-1 are the up rows matching gate rows 0 .. R-1
  const uint8_t *wrow[RR];
  const uint16_t *srow[RR];
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    const uint8_t *wv = v == 0 ? w : w2;
    const uint16_t *scales = reinterpret_cast<const uint16_t *>(wv + (uint64_t)n * k / 4u);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t row = min(row_base + r, n - 1u);
      wrow[v * R + r] = wv + (uint64_t)row * (k >> 2);
      srow[v * R + r] = scales + (uint64_t)row * G;
    }
  }

  // This thread's prep items.  Item order (m, group, field, half) makes
  // consecutive threads read consecutive 32-byte activation runs.  Threads
  // past the last item load that item's activations again (their loads stay
  // unconditional) but write nothing.
  uint32_t it_m[kPrep], it_cl[kPrep], it_j[kPrep], it_src[kPrep];
#pragma unroll
  for (int q = 0; q < kPrep; ++q) {
    const uint32_t it = min(tid + (uint32_t)(kThreads * q), (uint32_t)kItems - 1u);
    const uint32_t m = it / (4u * L), rr = it % (4u * L);
    const uint32_t h = rr & 1u, j = (rr >> 1) & 3u, gl = rr >> 3;
    it_m[q] = m;
    it_cl[q] = 2u * gl + h;
    it_j[q] = j;
    it_src[q] = m * k + 32u * j + 16u * h;  // element offset of the run within its 128-group
  }

  uint4 wq[D][RR];
  uint32_t sc[D][RR];
  uint4 av[kPrep][2];

#define BQMM_LOAD_W(slot, sl)                                                      \
  do {                                                                             \
    const uint32_t c_ = min((uint32_t)(sl) * L + li, C - 1u);                      \
    _Pragma("unroll") for (int r = 0; r < RR; ++r) {                               \
      wq[slot][r] = *reinterpret_cast<const uint4 *>(wrow[r] + 16u * c_);          \
      sc[slot][r] = srow[r][c_ >> 1];                                              \
    }                                                                              \
  } while (0)

#define BQMM_LOAD_A(regs, sl)                                                      \
  do {                                                                             \
    _Pragma("unroll") for (int q = 0; q < kPrep; ++q) {                            \
      const uint32_t c_ = min((uint32_t)(sl) * L + it_cl[q], C - 1u);              \
      const uint16_t *p_ = act + it_src[q] + 128u * (c_ >> 1);                     \
      regs[q][0] = *reinterpret_cast<const uint4 *>(p_);                           \
      regs[q][1] = *reinterpret_cast<const uint4 *>(p_ + 8);                       \
    }                                                                              \
  } while (0)

#define BQMM_PREP(regs, sl, buf)                                                   \
  do {                                                                             \
    _Pragma("unroll") for (int q = 0; q < kPrep; ++q) {                            \
      /* whole waves past the last item skip (kItems is a multiple of 64) */       \
      if (kItems % kThreads != 0 && tid + (uint32_t)(kThreads * q) >= (uint32_t)kItems) continue; \
      const bool live_ = (uint32_t)(sl) * L + it_cl[q] < C;                        \
      uint32_t Dw_[8] = {regs[q][0].x, regs[q][0].y, regs[q][0].z, regs[q][0].w,  \
                         regs[q][1].x, regs[q][1].y, regs[q][1].z, regs[q][1].w};  \
      _Pragma("unroll") for (int i = 0; i < 8; ++i) Dw_[i] = live_ ? Dw_[i] : 0u;  \
      uint32_t p_[8];                                                              \
      act_pairs(Dw_, p_);                                                          \
      const uint32_t j_ = it_j[q];                                                 \
      const float b_ = field_bias(Dw_, bias_weight(j_));                           \
      uint32_t *dst_ = lds + (buf) * kBuf + it_cl[q] * CS + it_m[q] * kRowDw;      \
      _Pragma("unroll") for (int i = 0; i < 4; ++i)                                \
        *reinterpret_cast<uint2 *>(dst_ + 8 * i + 2 * j_) =                        \
            make_uint2(p_[2 * i], p_[2 * i + 1]);                                  \
      dst_[32 + j_] = __float_as_uint(b_);                                         \
    }                                                                              \
  } while (0)

  const CodeConsts K = code_consts();
  float oacc[RR][M];
#pragma unroll
  for (int r = 0; r < RR; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) oacc[r][m] = 0.0f;

// One (word i, activation row m) unit: 8 activation pairs from LDS feed
// 8 R dot2.  The next unit's LDS reads are issued before this unit's dot2s.
// After each unit its accumulators pass through an empty asm that also
// redefines the LDS offset, so the reads of unit u + 2 cannot be hoisted above
// the dot2s of unit u: without it the compiler issues every read of the chunk
// up front (32 M registers).
#define BQMM_COMPUTE(slot, buf)                                                    \
  do {                                                                             \
    uint32_t off_ = (buf) * kBuf + li * CS;                                        \
    float acc_[RR][M];                                                              \
    _Pragma("unroll") for (int m = 0; m < M; ++m) {                                \
      const uint4 bq_ = *reinterpret_cast<const uint4 *>(lds + off_ + m * kRowDw + 32); \
      const float nb_ = -((__uint_as_float(bq_.x) + __uint_as_float(bq_.y)) +      \
                          (__uint_as_float(bq_.z) + __uint_as_float(bq_.w)));      \
      _Pragma("unroll") for (int r = 0; r < RR; ++r) acc_[r][m] = nb_;              \
    }                                                                              \
    uint4 pa_ = *reinterpret_cast<const uint4 *>(lds + off_);                      \
    uint4 pb_ = *reinterpret_cast<const uint4 *>(lds + off_ + 4);                  \
    uint32_t wp_[RR][8];                                                            \
    _Pragma("unroll") for (int u_ = 0; u_ < 4 * M; ++u_) {                         \
      const int i = u_ / M, m = u_ % M;                                            \
      if (m == 0) {                                                                \
        _Pragma("unroll") for (int r = 0; r < RR; ++r) {                            \
          const uint32_t x_ = (i == 0) ? wq[slot][r].x : (i == 1) ? wq[slot][r].y  \
                            : (i == 2) ? wq[slot][r].z : wq[slot][r].w;            \
          word_pairs(x_, K, wp_[r]);                                               \
        }                                                                          \
      }                                                                            \
      const uint32_t P_[8] = {pa_.x, pa_.y, pa_.z, pa_.w, pb_.x, pb_.y, pb_.z, pb_.w}; \
      if (u_ + 1 < 4 * M) {                                                        \
        const int i2 = (u_ + 1) / M, m2 = (u_ + 1) % M;                            \
        pa_ = *reinterpret_cast<const uint4 *>(lds + off_ + m2 * kRowDw + 8 * i2);     \
        pb_ = *reinterpret_cast<const uint4 *>(lds + off_ + m2 * kRowDw + 8 * i2 + 4); \
      }                                                                            \
      _Pragma("unroll") for (int r = 0; r < RR; ++r)                                \
        _Pragma("unroll") for (int qq = 0; qq < 8; ++qq)                           \
          acc_[r][m] = dot2(wp_[r][qq], P_[qq], acc_[r][m]);                       \
      _Pragma("unroll") for (int r = 0; r < RR; ++r)                                \
        asm volatile("" : "+v"(off_) : "v"(acc_[r][m]));                           \
    }                                                                              \
    _Pragma("unroll") for (int r = 0; r < RR; ++r) {                                \
      const float d_ = f16_bits_to_f32(sc[slot][r]);                               \
      _Pragma("unroll") for (int m = 0; m < M; ++m)                                \
        oacc[r][m] = fmaf(d_, acc_[r][m], oacc[r][m]);                             \
    }                                                                              \
  } while (0)

  // Prologue: activations of slices 0 and 1, then D slices of weights, so
  // that the loads pending at the loop entry are in the same order (the
  // activations of the next prep ahead of the weights) as at its back edge.
  {
    uint4 av0[kPrep][2];
    BQMM_LOAD_A(av0, 0);
    BQMM_LOAD_A(av, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < D; ++u) BQMM_LOAD_W(u, u);
    BQMM_PREP(av0, 0, 0);
  }
  __syncthreads();

  // Full groups of D slices.  Every load is unconditional (clamped past the
  // end): a load under a branch would be merged into its slot registers at
  // the join with a copy that waits for it, draining the prefetch.
  uint32_t s0 = 0;
  for (; s0 + D <= ns; s0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const uint32_t sl = s0 + u;
      BQMM_COMPUTE(u, sl & 1u);
      BQMM_PREP(av, sl + 1u, (sl + 1u) & 1u);
      BQMM_LOAD_A(av, sl + 2u);
      __builtin_amdgcn_sched_barrier(0);  // keep the activation loads ahead
      BQMM_LOAD_W(u, sl + D);
      __syncthreads();
    }
  }
  // The last ns - s0 < D slices: their weights and activations are already
  // loaded, so these steps issue no loads.
#pragma unroll
  for (int u = 0; u < D - 1; ++u) {
    const uint32_t sl = s0 + u;
    if (sl < ns) {
      BQMM_COMPUTE(u, sl & 1u);
      if (sl + 1u < ns) {
        BQMM_PREP(av, sl + 1u, (sl + 1u) & 1u);
        __syncthreads();
      }
    }
  }
#undef BQMM_LOAD_W
#undef BQMM_LOAD_A
#undef BQMM_PREP
#undef BQMM_COMPUTE

#pragma unroll
  for (int r = 0; r < RR; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m)
      oacc[r][m] = (L == 16) ? row16_sum(oacc[r][m]) : half_wave_sum(oacc[r][m]);
  if (li == (uint32_t)L - 1u) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t row = row_base + r;
      if (row < n) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
          uint32_t h = f32_to_bf16_rne(oacc[r][m]);
          if (NW == 2) {
            // gate and up rounded to bf16 as separate GEMV outputs would be
            const float g = bf16_to_f32(h), u = bf16_to_f32(f32_to_bf16_rne(oacc[R + r][m]));
            h = f32_to_bf16_rne(silu_mul_f32(g, u));
          }
          out[(uint64_t)m * n + row] = (uint16_t)h;
        }
      }
    }
  }
}

// ---- whole-vector pipelined kernel, m = 1..3 ------------------------------
//
// For the verify batches (and m = 1) when the activations of all M rows fit in
// LDS: they are prepared once per workgroup (no per-slice barriers), and a
// lane then walks its chunks li, li + G, ... of R rows with the next chunk's
// weight loads in flight while the current one is computed.  Prep items are
// (chunk, activation row): the four 32-byte runs of a chunk's 64 values are
// loaded together (eight 16-byte loads), so a workgroup's prep takes few
// memory round trips.  LDS per chunk as in the slice kernel (word-major
// pairs, then the four partial biases; chunks padded so that 16 consecutive
// chunks read by one instruction hit distinct bank quads); chunks past k hold
// zero activations and biases, so their clamped weight loads add 0.
template <int M, int G, int R, int NW, int PD>
__global__ __launch_bounds__(kThreads) void q2_0_gemvp_kernel(const uint16_t *__restrict__ act,
                                                              const uint8_t *__restrict__ w,
                                                              const uint8_t *__restrict__ w2,
                                                              uint16_t *__restrict__ out, uint32_t n,
                                                              uint32_t k) {
  static_assert(G == 16 || G == 32, "lane group of 16 or 32");
  static_assert(NW == 1 || NW == 2, "one weight, or gate and up");
  static_assert(PD == 2 || PD == 3, "two or three weight register sets");
  constexpr int RR = NW * R;
  constexpr int CS = gemvm_chunk_dwords(M);
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  const uint32_t C = k >> 6, Gk = k >> 7;
  const uint32_t tid = threadIdx.x, li = tid % G, grp = tid / G;
  const uint32_t iters = (C + G - 1) / G, Cpad = iters * G;
  const uint32_t row_base = blockIdx.x * (kThreads / G * R) + grp * R;

  const uint8_t *wrow[RR];
  const uint16_t *srow[RR];
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    const uint8_t *wv = v == 0 ? w : w2;
    const uint16_t *scales = reinterpret_cast<const uint16_t *>(wv + (uint64_t)n * k / 4u);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t row = min(row_base + r, n - 1u);
      wrow[v * R + r] = wv + (uint64_t)row * (k >> 2);
      srow[v * R + r] = scales + (uint64_t)row * Gk;
    }
  }
  auto load_unit = [&](uint32_t it, uint4 (&wq)[RR], uint32_t (&sc)[RR]) {
    const uint32_t c = min(li + G * it, C - 1u);
#pragma unroll
    for (int r = 0; r < RR; ++r) {
      wq[r] = *reinterpret_cast<const uint4 *>(wrow[r] + 16u * c);
      sc[r] = srow[r][c >> 1];
    }
  };

  // prep item (chunk c, activation row m): runs j = 0..3 of 16 values at
  // k = 128 (c / 2) + 32 j + 16 (c % 2)
  const uint32_t items = Cpad * M;
  auto load_item = [&](uint32_t item, uint4 (&v)[8]) {
    const uint32_t c = min(item / M, C - 1u), m = item % M;
    const uint16_t *src = act + (uint64_t)m * k + 128u * (c >> 1) + 16u * (c & 1u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = *reinterpret_cast<const uint4 *>(src + 32 * j);
      v[2 * j + 1] = *reinterpret_cast<const uint4 *>(src + 32 * j + 8);
    }
  };
  auto prep_item = [&](uint32_t item, const uint4 (&v)[8]) {
    const uint32_t c = item / M, m = item % M;
    const bool live = c < C;
    uint32_t *dst = smem + c * CS + m * kRowDw;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t D[8] = {v[2 * j].x, v[2 * j].y, v[2 * j].z, v[2 * j].w,
                       v[2 * j + 1].x, v[2 * j + 1].y, v[2 * j + 1].z, v[2 * j + 1].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) D[i] = live ? D[i] : 0u;
      uint32_t p[8];
      act_pairs(D, p);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<uint2 *>(dst + 8 * i + 2 * j) = make_uint2(p[2 * i], p[2 * i + 1]);
      dst[32 + j] = __float_as_uint(field_bias(D, bias_weight((uint32_t)j)));
    }
  };

  uint4 wq[PD][RR];
  uint32_t sc[PD][RR];
  {
    // the first item's activation loads go out before the first weight loads
    uint4 v[8];
    const uint32_t first = min(tid, items - 1u);
    load_item(first, v);
#pragma unroll
    for (int p = 0; p + 1 < PD; ++p) load_unit(p, wq[p], sc[p]);
    if (tid < items) prep_item(first, v);
  }
  for (uint32_t item = tid + kThreads; item < items; item += kThreads) {
    uint4 v[8];
    load_item(item, v);
    prep_item(item, v);
  }
  __syncthreads();

  const CodeConsts K = code_consts();
  float oacc[RR][M];
#pragma unroll
  for (int r = 0; r < RR; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) oacc[r][m] = 0.0f;

  // One chunk: per (word i, activation row m) 8 pairs from LDS feed 8 R dot2s;
  // the next unit's reads are issued before this unit's dot2s, and an empty
  // asm on the accumulators keeps the compiler from hoisting every read of the
  // chunk (as in the slice kernel).
  auto compute = [&](uint32_t it, const uint4 (&wq)[RR], const uint32_t (&sc)[RR]) {
    uint32_t off = (li + G * it) * CS;
    float acc[RR][M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint4 bq = *reinterpret_cast<const uint4 *>(smem + off + m * kRowDw + 32);
      const float nb = -((__uint_as_float(bq.x) + __uint_as_float(bq.y)) +
                         (__uint_as_float(bq.z) + __uint_as_float(bq.w)));
#pragma unroll
      for (int r = 0; r < RR; ++r) acc[r][m] = nb;
    }
    uint4 pa = *reinterpret_cast<const uint4 *>(smem + off);
    uint4 pb = *reinterpret_cast<const uint4 *>(smem + off + 4);
    uint32_t wp[RR][8];
#pragma unroll
    for (int u = 0; u < 4 * M; ++u) {
      const int i = u / M, m = u % M;
      if (m == 0) {
#pragma unroll
        for (int r = 0; r < RR; ++r) {
          const uint32_t x = (i == 0) ? wq[r].x : (i == 1) ? wq[r].y : (i == 2) ? wq[r].z : wq[r].w;
          word_pairs(x, K, wp[r]);
        }
      }
      const uint32_t P[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
      if (u + 1 < 4 * M) {
        const int i2 = (u + 1) / M, m2 = (u + 1) % M;
        pa = *reinterpret_cast<const uint4 *>(smem + off + m2 * kRowDw + 8 * i2);
        pb = *reinterpret_cast<const uint4 *>(smem + off + m2 * kRowDw + 8 * i2 + 4);
      }
#pragma unroll
      for (int r = 0; r < RR; ++r)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[r][m] = dot2(wp[r][q], P[q], acc[r][m]);
#pragma unroll
      for (int r = 0; r < RR; ++r) asm volatile("" : "+v"(off) : "v"(acc[r][m]));
    }
#pragma unroll
    for (int r = 0; r < RR; ++r) {
      const float d = f16_bits_to_f32(sc[r]);
#pragma unroll
      for (int m = 0; m < M; ++m) oacc[r][m] = fmaf(d, acc[r][m], oacc[r][m]);
    }
  };

  if constexpr (PD == 2) {
    // two register sets alternate; the last one or two chunks are peeled so
    // that every prefetch is unconditional, and the scheduling barriers keep
    // each prefetch above the wait for the chunk being computed
    uint32_t it = 0;
    for (; it + 2 < iters; it += 2) {
      load_unit(it + 1, wq[1], sc[1]);
      __builtin_amdgcn_sched_barrier(0);
      compute(it, wq[0], sc[0]);
      load_unit(it + 2, wq[0], sc[0]);
      __builtin_amdgcn_sched_barrier(0);
      compute(it + 1, wq[1], sc[1]);
    }
    if (it + 1 < iters) {
      load_unit(it + 1, wq[1], sc[1]);
      __builtin_amdgcn_sched_barrier(0);
      compute(it, wq[0], sc[0]);
      compute(it + 1, wq[1], sc[1]);
    } else {
      compute(it, wq[0], sc[0]);
    }
  } else {
    // three sets rotate (long rows): unit it + 2 is loaded while unit it is
    // computed; loads past the last unit read the clamped last chunk and are
    // not computed
    for (uint32_t it = 0; it < iters; it += PD) {
#pragma unroll
      for (int p = 0; p < PD; ++p) {
        load_unit(it + p + PD - 1, wq[(p + PD - 1) % PD], sc[(p + PD - 1) % PD]);
        __builtin_amdgcn_sched_barrier(0);
        if (it + p < iters) compute(it + p, wq[p], sc[p]);
      }
    }
  }

#pragma unroll
  for (int r = 0; r < RR; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) oacc[r][m] = (G == 16) ? row16_sum(oacc[r][m]) : half_wave_sum(oacc[r][m]);
  if (li == (uint32_t)G - 1u) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t row = row_base + r;
      if (row < n) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
          uint32_t h = f32_to_bf16_rne(oacc[r][m]);
          if (NW == 2) {
            const float g = bf16_to_f32(h), u = bf16_to_f32(f32_to_bf16_rne(oacc[R + r][m]));
            h = f32_to_bf16_rne(silu_mul_f32(g, u));
          }
          out[(uint64_t)m * n + row] = (uint16_t)h;
        }
      }
    }
  }
}

// Launch shape (measured on the FFN shapes, m = 1..3): 16-lane groups; the
// single kernel serves m rows per lane for m activation rows (each LDS read
// then feeds m x m products), the fused gate/up kernel one row of each weight.
// Against the slice kernel: gate [17408, 5120] m = 1/2/3 8.8/11.8/14.6 us
// (was 10.3/13.5/16.1), down m = 1 12.0 us (was 16.2), fused gate/up m = 1/2/3
// 13.6/18.2/23.7 us (was 19.6/25.3/30.0).  32-lane groups were slower at
// m >= 2; with more than 64 KB of LDS (down at m = 2, 3) it is slower than
// the slice kernel, which keeps those.
#ifndef BQMM_GEMVP_G
#define BQMM_GEMVP_G 16
#endif
#ifndef BQMM_GEMVP_MAX_LDS
#define BQMM_GEMVP_MAX_LDS 65536
#endif
constexpr uint32_t kMaxLdsP = BQMM_GEMVP_MAX_LDS;

// LDS bytes of the whole-vector kernel for m rows and k (0 if m > 3)
__host__ __device__ inline uint32_t gemvp_lds_bytes(uint32_t m, uint32_t k) {
  if (m < 1 || m > 3) return 0;
  const uint32_t C = k >> 6, Cpad = (C + BQMM_GEMVP_G - 1) / BQMM_GEMVP_G * BQMM_GEMVP_G;
  const uint32_t cs = m == 1 ? gemvm_chunk_dwords(1) : (m == 2 ? gemvm_chunk_dwords(2) : gemvm_chunk_dwords(3));
  return Cpad * cs * 4u;
}

template <int M, int NW, int PD>
hipError_t launch_gemvp_pd(const void *act, const void *w, const void *w2, void *out, uint32_t n, uint32_t k,
                           hipStream_t s) {
  constexpr int G = BQMM_GEMVP_G, R = NW == 2 ? 1 : M;
  const uint32_t lds = gemvp_lds_bytes(M, k);
  if (lds > 65536u) {
    const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void *>(q2_0_gemvp_kernel<M, G, R, NW, PD>),
                                            (int)kMaxLdsP);
    if (e != hipSuccess) return e;
  }
  constexpr uint32_t rows = kThreads / G * R;
  const uint32_t blocks = (n + rows - 1) / rows;
  hipLaunchKernelGGL((q2_0_gemvp_kernel<M, G, R, NW, PD>), dim3(blocks), dim3(kThreads), lds, s,
                     static_cast<const uint16_t *>(act), static_cast<const uint8_t *>(w),
                     static_cast<const uint8_t *>(w2), static_cast<uint16_t *>(out), n, k);
  return hipGetLastError();
}

// A third weight register set pays off for one activation row and long rows:
// down [5120, 17408] m = 1 (17 chunks per lane) 12.0 -> 11.3 us, while every
// k = 5120 shape (5 chunks per lane) measured slower with it.
template <int M, int NW>
hipError_t launch_gemvp(const void *act, const void *w, const void *w2, void *out, uint32_t n, uint32_t k,
                        hipStream_t s) {
  if constexpr (M == 1 && NW == 1) {
    if ((k >> 6) >= 12u * BQMM_GEMVP_G) return launch_gemvp_pd<M, NW, 3>(act, w, w2, out, n, k, s);
  }
  return launch_gemvp_pd<M, NW, 2>(act, w, w2, out, n, k, s);
}

// Launch shapes (measured): wide outputs (gate/up, n = 17408) take 16-lane
// groups of three rows (48 rows per workgroup, one slice = 1024 k); narrow
// outputs with a long k (down, n = 5120, k = 17408) take 32-lane groups of four
// rows (32 rows per workgroup).  More rows per lane amortize the activation
// prep and the LDS reads over more weight bytes.
#ifndef BQMM_GEMVM_WIDE_R
#define BQMM_GEMVM_WIDE_R 3
#endif
#ifndef BQMM_GEMVM_WIDE_L
#define BQMM_GEMVM_WIDE_L 16
#endif
#ifndef BQMM_GEMVM_NARROW_R
#define BQMM_GEMVM_NARROW_R 3
#endif
#ifndef BQMM_GEMVM_NARROW_L
#define BQMM_GEMVM_NARROW_L 32
#endif
#ifndef BQMM_GEMVM_FUSED_R
#define BQMM_GEMVM_FUSED_R 2
#endif
#ifndef BQMM_GEMVM_SLOTS
#define BQMM_GEMVM_SLOTS 3
#endif
#ifndef BQMM_GEMVM_WIDE_N
#define BQMM_GEMVM_WIDE_N 8192
#endif

template <int M, int R, int L, int NW>
hipError_t launch_gemvm_shape(const void *act, const void *w, const void *w2, void *out, uint32_t n,
                              uint32_t k, hipStream_t s) {
  constexpr uint32_t rows = (kThreads / L) * R;
  const uint32_t blocks = (n + rows - 1) / rows;
  hipLaunchKernelGGL((q2_0_gemvm_kernel<M, R, L, BQMM_GEMVM_SLOTS, NW>), dim3(blocks), dim3(kThreads), 0, s,
                     static_cast<const uint16_t *>(act), static_cast<const uint8_t *>(w),
                     static_cast<const uint8_t *>(w2), static_cast<uint16_t *>(out), n, k);
  return hipGetLastError();
}

// The lane-group width L follows n in the same way for the single and the
// fused (gate + up) kernel, so that each output row is summed in the same
// order by both and the fused result equals GEMV, GEMV, silu_mul bit for bit.
template <int M>
hipError_t launch_gemvm(const void *act, const void *w, void *out, uint32_t n, uint32_t k,
                        hipStream_t s) {
  if (n >= BQMM_GEMVM_WIDE_N)
    return launch_gemvm_shape<M, BQMM_GEMVM_WIDE_R, BQMM_GEMVM_WIDE_L, 1>(act, w, nullptr, out, n, k, s);
  return launch_gemvm_shape<M, BQMM_GEMVM_NARROW_R, BQMM_GEMVM_NARROW_L, 1>(act, w, nullptr, out, n, k, s);
}

// Two rows of each weight per lane up to m = 5; one from m = 6 on (reached
// only for k beyond the matrix-core kernel's limit), where the
// accumulators of 4 rows x m columns would crowd out the weight prefetch.
template <int M>
hipError_t launch_gemvm_gate_up(const void *act, const void *wg, const void *wu, void *out, uint32_t n,
                                uint32_t k, hipStream_t s) {
  constexpr int R = M >= 6 ? 1 : BQMM_GEMVM_FUSED_R;
  if (n >= BQMM_GEMVM_WIDE_N)
    return launch_gemvm_shape<M, R, BQMM_GEMVM_WIDE_L, 2>(act, wg, wu, out, n, k, s);
  return launch_gemvm_shape<M, R, BQMM_GEMVM_NARROW_L, 2>(act, wg, wu, out, n, k, s);
}

}  // namespace

#ifndef BQMM_GEMVP_ENABLE
#define BQMM_GEMVP_ENABLE 1
#endif
#ifndef BQMM_GEMVP_M1_MIN_K
#define BQMM_GEMVP_M1_MIN_K 4096
#endif

// The whole-vector kernel serves m <= 3 below the matrix-core threshold where
// its LDS fits (and m = 1 from BQMM_GEMVP_M1_MIN_K on); the single and fused
// dispatch make the same choice.
inline bool use_gemvp(uint32_t m, uint32_t k) {
  if (!BQMM_GEMVP_ENABLE || m > 3 || m >= kMinMMfma) return false;
  if (m == 1 && k < BQMM_GEMVP_M1_MIN_K) return false;
  return gemvp_lds_bytes(m, k) <= kMaxLdsP;
}

// The matrix-core kernel serves m >= kMinMMfma where the fused gate/up
// launch's staged scales fit its LDS (the stricter of the two launches), so
// that the single and the fused call take the same kernel for every shape.
inline bool use_gemv_mfma(uint32_t m, uint32_t n, uint32_t k) {
  return m >= kMinMMfma && q2_0_gemv_mfma_fits(n, k, 2);
}

hipError_t launch_q2_0_gemv(const void *act, const void *w, void *out, uint32_t m, uint32_t n,
                            uint32_t k, hipStream_t s) {
  if (use_gemvp(m, k)) {
    switch (m) {
      case 1: return launch_gemvp<1, 1>(act, w, nullptr, out, n, k, s);
      case 2: return launch_gemvp<2, 1>(act, w, nullptr, out, n, k, s);
#if BQMM_GEMV_MIN_M_MFMA > 3
      default: return launch_gemvp<3, 1>(act, w, nullptr, out, n, k, s);
#else
      default: return hipErrorInvalidValue;  // m = 3 runs on the matrix-core kernel
#endif
    }
  }
  if (m == 1 && k <= kMaxK1) {
    const uint32_t blocks = (n + 8 * kRowsPerLane - 1) / (8 * kRowsPerLane);
    const size_t lds = (size_t)(k >> 6) * kChunkStride * 4u;  // 72 KB at kMaxK1
    if (lds > 65536u) {
      const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void *>(q2_0_gemv1_kernel), (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(q2_0_gemv1_kernel, dim3(blocks), dim3(kThreads), lds, s,
                       static_cast<const uint16_t *>(act), static_cast<const uint8_t *>(w),
                       static_cast<uint16_t *>(out), n, k);
    return hipGetLastError();
  }
  // From m = 3 on the per-code multiply-adds outweigh the code unpacking and
  // the matrix-core kernel is faster (its LDS bounds k).  Measured on the FFN
  // shapes (A/B on one machine, cold): at m = 3 down [5120, 17408] 20.9 -> 15.0 us
  // and gate [17408, 5120] 14.0 -> 12.0 us, the fused gate/up 23.0 -> 23.5 us
  // (2% slower, but it has to take the single call's kernel); at m = 2 the
  // vector kernels stay ahead (gate 11.4 against 11.8 us, down 13.4 against
  // 14.5, fused 17.3 against 23.1).
  if (use_gemv_mfma(m, n, k)) return launch_q2_0_gemv_mfma(act, w, out, m, n, k, s);
  switch (m) {
    case 1: return launch_gemvm<1>(act, w, out, n, k, s);
    case 2: return launch_gemvm<2>(act, w, out, n, k, s);
    case 3: return launch_gemvm<3>(act, w, out, n, k, s);
    case 4: return launch_gemvm<4>(act, w, out, n, k, s);
    case 5: return launch_gemvm<5>(act, w, out, n, k, s);
    case 6: return launch_gemvm<6>(act, w, out, n, k, s);
    case 7: return launch_gemvm<7>(act, w, out, n, k, s);
    case 8: return launch_gemvm<8>(act, w, out, n, k, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_q2_0_gemv_gate_up_silu(const void *act, const void *w_gate, const void *w_up,
                                         void *out, uint32_t m, uint32_t n, uint32_t k,
                                         hipStream_t s) {
  // One launch for every m, on the kernel the single GEMV uses for that m, so
  // the result equals GEMV, GEMV, silu_mul.
  if (use_gemvp(m, k)) {
    switch (m) {
      case 1: return launch_gemvp<1, 2>(act, w_gate, w_up, out, n, k, s);
      case 2: return launch_gemvp<2, 2>(act, w_gate, w_up, out, n, k, s);
#if BQMM_GEMV_MIN_M_MFMA > 3
      default: return launch_gemvp<3, 2>(act, w_gate, w_up, out, n, k, s);
#else
      default: return hipErrorInvalidValue;  // m = 3 runs on the matrix-core kernel
#endif
    }
  }
  if (use_gemv_mfma(m, n, k))
    return launch_q2_0_gemv_mfma_gate_up(act, w_gate, w_up, out, m, n, k, s);
  switch (m) {
    case 1: return launch_gemvm_gate_up<1>(act, w_gate, w_up, out, n, k, s);
    case 2: return launch_gemvm_gate_up<2>(act, w_gate, w_up, out, n, k, s);
    case 3: return launch_gemvm_gate_up<3>(act, w_gate, w_up, out, n, k, s);
    case 4: return launch_gemvm_gate_up<4>(act, w_gate, w_up, out, n, k, s);
    case 5: return launch_gemvm_gate_up<5>(act, w_gate, w_up, out, n, k, s);
    case 6: return launch_gemvm_gate_up<6>(act, w_gate, w_up, out, n, k, s);
    case 7: return launch_gemvm_gate_up<7>(act, w_gate, w_up, out, n, k, s);
    case 8: return launch_gemvm_gate_up<8>(act, w_gate, w_up, out, n, k, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bqmm

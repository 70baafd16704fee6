// Q2_0 GEMV for decode (m = 1) and small verify batches (m = 2..8).
//
// [page layers/qwen3_ssm/init.rs, kernel q2_0_gemv_vec; page
//  layers/dense_ffn_decode_batch.rs, fn forward_km_q2: q2_0_gemv_vec_batchm on
//  the bf16 activations, output bf16.]
//
// out[i][r] = sum_k a[i][k] * d[r][g] * (c - 2), accumulated in fp32.
// A bandwidth kernel: the packed weight (2.125 bits per weight) is streamed
// once with 16-byte loads; no matrix cores.  16 lanes share one weight row;
// lane L owns the 16-byte half-groups L, L+16, ... of the row, i.e. 64 codes
// per load: for field j of byte t the code belongs to k = 128g + 32j + 16h + t.
#include "bqmm_internal.h"

namespace bqmm {
namespace {

constexpr int kLanesPerRow = 16;
constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / kLanesPerRow;

template <int M>
__global__ __launch_bounds__(kThreads) void q2_0_gemv_kernel(const uint16_t *__restrict__ act,
                                                             const uint8_t *__restrict__ w,
                                                             uint16_t *__restrict__ out,
                                                             uint32_t n, uint32_t k) {
  const uint32_t sub = threadIdx.x % kLanesPerRow;
  const uint32_t row = blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  const uint32_t chunks = k / 64u;  // 16-byte half-groups per row
  const uint16_t *scales = reinterpret_cast<const uint16_t *>(w + (uint64_t)n * k / 4u);

  float acc[M];
#pragma unroll
  for (int i = 0; i < M; ++i) acc[i] = 0.0f;

  if (row < n) {
    const uint8_t *wrow = w + (uint64_t)row * (k / 4u);
    for (uint32_t c = sub; c < chunks; c += kLanesPerRow) {
      const uint32_t g = c >> 1, h = c & 1u;
      const uint4 q = *reinterpret_cast<const uint4 *>(wrow + 16u * c);
      const float d = f16_bits_to_f32(scales[(uint64_t)row * (k / 128u) + g]);
      const uint32_t words[4] = {q.x, q.y, q.z, q.w};
      float part[M];
#pragma unroll
      for (int i = 0; i < M; ++i) part[i] = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t kbase = 128u * g + 32u * j + 16u * h;
#pragma unroll
        for (int i = 0; i < M; ++i) {
          const uint4 a0 = *reinterpret_cast<const uint4 *>(act + (uint64_t)i * k + kbase);
          const uint4 a1 = *reinterpret_cast<const uint4 *>(act + (uint64_t)i * k + kbase + 8);
          const uint32_t av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const uint32_t code = (words[t / 4] >> (8 * (t % 4) + 2 * j)) & 3u;
            const float wv = (float)((int)code - 2);
            const float av_f = (t & 1) ? __uint_as_float(av[t / 2] & 0xFFFF0000u)
                                       : __uint_as_float(av[t / 2] << 16);
            part[i] = fmaf(wv, av_f, part[i]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < M; ++i) acc[i] = fmaf(d, part[i], acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < M; ++i) {
#pragma unroll
    for (int off = kLanesPerRow / 2; off > 0; off >>= 1) acc[i] += __shfl_xor(acc[i], off);
  }
  if (row < n && sub == 0) {
#pragma unroll
    for (int i = 0; i < M; ++i) out[(uint64_t)i * n + row] = (uint16_t)f32_to_bf16_rne(acc[i]);
  }
}

// ---- m = 1 decode kernel ---------------------------------------------------
//
// Each lane keeps one fixed 16-byte chunk position c of the weight rows (64
// codes: half of a 128-group) and serves kRowsPerLane rows; a half-wave (32
// lanes) covers 32 consecutive chunks of a row.  The activation slice of every
// chunk is prepared once per workgroup in LDS:
//   * pairs: for the 16-byte word i of a chunk and field j, the codes of bytes
//     (0, 2) and (1, 3) of the word pair with activations (t, t+2), so the
//     activations are permuted into those pairs;
//   * the code field j sits at bits 2j of each byte; OR-ing a masked field into
//     the mantissa of bf16 1.0 gives 1 + c * 2^-e_j (e = 7, 5, 3 for j = 0..2;
//     field 3 is shifted down one bit, e = 2), exact in bf16, with one
//     v_and_or_b32 per pair of codes;
//   * the activation of field j is stored with its exponent raised by e_j
//     (a' = a * 2^e_j, a packed 16-bit add; exact), so every product
//     (1 + c 2^-e) * a' = a' + c * a and one v_dot2_f32_bf16 handles two codes;
//   * four partial biases per chunk, sum a' (1 + 2 * 2^-e) over each field, so
//     that sum_k (c - 2) a = dot - bias.
// Per row and chunk: 12 bit ops + 32 dot2 + 1 fma for 64 codes.  The weight
// loads of the first slice are issued before the activation prep, which is
// spread over one lane per (chunk, field) and runs while they are in flight.
// Row sums over the 32 lanes of a half-wave use DPP adds (no LDS round trip).
// Activations are assumed below 2^120 in magnitude (the exponent add must not
// overflow).

#ifndef BQMM_GEMV_ROWS
#define BQMM_GEMV_ROWS 3
#endif
constexpr int kRowsPerLane = BQMM_GEMV_ROWS;
constexpr int kChunkStride = 36;  // dwords per chunk in LDS: 32 pairs, 4 partial biases
constexpr uint32_t kMaxK1 = 32768;

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, a), __builtin_bit_cast(v2bf, b), c, false);
}

__device__ __forceinline__ uint32_t add_u16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(v2u16, a) + __builtin_bit_cast(v2u16, b));
}

__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t bits) {
  return (x & mask) | bits;
}

// A constant materialized in a VGPR and opaque to the optimizer.  gfx9 VOP3
// encodings take no literal, so with literal masks the compiler splits
// (x & m) | b into v_and_b32 + v_or_b32; with the masks in VGPRs it selects
// one v_and_or_b32 per code pair.
__device__ __forceinline__ uint32_t vconst(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

// x plus the value DPP moves into this lane (rows not in row_mask add 0).
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_add(float x) {
  const int moved = __builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, kRowMask, 0xF, false);
  return x + __int_as_float(moved);
}

// Sum over each half-wave (lanes 0..31, 32..63); the total lands in lanes
// 16..31 and 48..63.
__device__ __forceinline__ float half_wave_sum(float x) {
  x = dpp_add<0xB1, 0xF>(x);   // quad_perm [1,0,3,2]: xor 1
  x = dpp_add<0x4E, 0xF>(x);   // quad_perm [2,3,0,1]: xor 2
  x = dpp_add<0x124, 0xF>(x);  // row_ror:4
  x = dpp_add<0x128, 0xF>(x);  // row_ror:8 -> every lane holds its 16-lane row sum
  x = dpp_add<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
  return x;
}

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
    const uint32_t e = (j == 0) ? 7u : (j == 1) ? 5u : (j == 2) ? 3u : 2u;
    const uint32_t add = (e << 7) | (e << 23);
    // bf16 of 1 + 2 * 2^-e: 1 + 2^-6, 1 + 2^-4, 1 + 2^-2, 1.5
    const uint32_t onep = (j == 0) ? 0x3F823F82u : (j == 1) ? 0x3F883F88u : (j == 2) ? 0x3FA03FA0u : 0x3FC03FC0u;
    uint32_t p[8];
    float b = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[2 * i] = add_u16x2(__builtin_amdgcn_perm(D[2 * i + 1], D[2 * i], 0x05040100u), add);
      p[2 * i + 1] = add_u16x2(__builtin_amdgcn_perm(D[2 * i + 1], D[2 * i], 0x07060302u), add);
      b = dot2(p[2 * i], onep, b);
      b = dot2(p[2 * i + 1], onep, b);
    }
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

  const uint32_t MAGIC = vconst(0x3F803F80u);  // bf16 1.0 in both halves
  const uint32_t M0 = vconst(0x00030003u), M1 = vconst(0x000C000Cu), M2 = vconst(0x00300030u),
                 M3 = vconst(0x00600060u);
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
          const uint32_t x = words[i], x8 = x >> 8, x1 = x >> 1, x9 = x >> 9;
          acc = dot2(and_or(x, M0, MAGIC), P[2 * i], acc);
          acc = dot2(and_or(x8, M0, MAGIC), P[2 * i + 1], acc);
          acc = dot2(and_or(x, M1, MAGIC), P[8 + 2 * i], acc);
          acc = dot2(and_or(x8, M1, MAGIC), P[8 + 2 * i + 1], acc);
          acc = dot2(and_or(x, M2, MAGIC), P[16 + 2 * i], acc);
          acc = dot2(and_or(x8, M2, MAGIC), P[16 + 2 * i + 1], acc);
          acc = dot2(and_or(x1, M3, MAGIC), P[24 + 2 * i], acc);
          acc = dot2(and_or(x9, M3, MAGIC), P[24 + 2 * i + 1], acc);
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

template <int M>
hipError_t launch_m(const void *act, const void *w, void *out, uint32_t n, uint32_t k,
                    hipStream_t s) {
  const uint32_t blocks = (n + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(q2_0_gemv_kernel<M>, dim3(blocks), dim3(kThreads), 0, s,
                     static_cast<const uint16_t *>(act), static_cast<const uint8_t *>(w),
                     static_cast<uint16_t *>(out), n, k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_q2_0_gemv(const void *act, const void *w, void *out, uint32_t m, uint32_t n,
                            uint32_t k, hipStream_t s) {
  if (m == 1 && k <= kMaxK1) {
    const uint32_t blocks = (n + 8 * kRowsPerLane - 1) / (8 * kRowsPerLane);
    const size_t lds = (size_t)(k >> 6) * kChunkStride * 4u;
    hipLaunchKernelGGL(q2_0_gemv1_kernel, dim3(blocks), dim3(kThreads), lds, s,
                       static_cast<const uint16_t *>(act), static_cast<const uint8_t *>(w),
                       static_cast<uint16_t *>(out), n, k);
    return hipGetLastError();
  }
  switch (m) {
    case 1: return launch_m<1>(act, w, out, n, k, s);
    case 2: return launch_m<2>(act, w, out, n, k, s);
    case 3: return launch_m<3>(act, w, out, n, k, s);
    case 4: return launch_m<4>(act, w, out, n, k, s);
    case 5: return launch_m<5>(act, w, out, n, k, s);
    case 6: return launch_m<6>(act, w, out, n, k, s);
    case 7: return launch_m<7>(act, w, out, n, k, s);
    case 8: return launch_m<8>(act, w, out, n, k, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bqmm

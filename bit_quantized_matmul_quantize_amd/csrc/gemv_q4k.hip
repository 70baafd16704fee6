// Q4_K GEMV for decode (m = 1): out[r] = sum_k a[k] * w[r][k], fp32
// accumulation, bf16 out, with w = d * sc_j * q - dmin * m_j per 32-weight
// sub-block j of a 256-weight super-block.
//
// [page layers/ops/q4k_mmq.rs: block_q4_K of 256 weights in 144 bytes and
//  fn q4k_mmq_gemm, C = A x W^T; the decode form multiplies the bf16
//  activations directly, as the Q2_0 decode GEMV does (page
//  layers/qwen3_ssm/init.rs, q2_0_gemv_vec).]
//
// Super-block layout: fp16 d, fp16 dmin, 12 bytes of 6-bit sub-scales and
// sub-mins, then 128 code bytes; byte 16 + 32t + i holds weight 64t + i in
// its low nibble and 64t + 32 + i in its high nibble.  A "unit" (t, super-
// block) is therefore 64 consecutive weights: sub-block 2t in the low
// nibbles and 2t + 1 in the high nibbles of the same 32 bytes.
//
// Codes become bf16 without a conversion: a nibble OR-ed into the mantissa of
// bf16 128.0 (0x4300) gives exactly 128 + q.  One v_and_or_b32 builds two
// such values from bytes 0 and 2 of a word (low nibbles); shifts by 8, 4 and
// 12 give bytes 1/3 and the high nibbles.  The activations are stored in LDS
// permuted into the matching pairs (4i, 4i+2), (4i+1, 4i+3), so one
// v_dot2_f32_bf16 adds (128 + q) a + (128 + q') a'.  Per sub-block the LDS
// also holds B = -128 * sum(a): the dot chain starts from B and ends at
// sum(q a), and the same B gives the min term, since
//   d sc sum(q a) - dmin m sum(a) = d sc (chain) + (dmin / 128) m B.
//
// Work split: the whole activation vector is prepared once per workgroup in
// LDS (36 dwords per unit: 16 pairs per sub-block, the two B, padding that
// keeps 16 consecutive units on distinct bank quads); beyond k = 65536
// (1024 units, 147 KB) it is prepared and consumed 1024 units at a time, with
// a barrier between chunks, in a second instantiation of the kernel.  A group of G lanes
// serves R rows; lane li takes units li, li + G, ...; since G is a multiple
// of 4, the lane's chunk t = li % 4 is fixed and so are its scale-field
// positions.  Per row and unit a lane loads the 16-byte header and the two
// 16-byte halves of its 32 code bytes; the next unit's loads are issued
// before the current unit is computed.
#include "gemv_common.h"

namespace bqmm {
namespace {

constexpr int kThreads = 256;
constexpr int kUnitDw = 36;                 // LDS dwords per unit
constexpr uint32_t kChunkUnits = 1024;      // units staged in LDS at a time: 147 KB, k = 65536
constexpr uint32_t kMagic128 = 0x43004300u;  // bf16 128.0 in both halves

struct UnitLoads {
  uint4 h, c0, c1;  // header, code bytes 0..15 and 16..31 of the unit
};

// kChunked: k > 65536, the activation vector staged one chunk of 1024 units
// at a time (otherwise in one piece, as a single chunk).
template <int G, int R, bool kChunked>
__global__ __launch_bounds__(kThreads) void q4k_gemv1_kernel(const uint16_t *__restrict__ act,
                                                             const uint8_t *__restrict__ w,
                                                             uint16_t *__restrict__ out, uint32_t n,
                                                             uint32_t k) {
  static_assert(G % 4 == 0 && kThreads % G == 0, "lane groups hold whole super-blocks");
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  const uint32_t tid = threadIdx.x;
  const uint32_t li = tid % G, grp = tid / G;
  const uint32_t nsb = k >> 8, U = nsb * 4u;
  uint32_t ub = 0;  // first unit of the chunk staged in LDS
  const uint32_t row_base = blockIdx.x * (kThreads / G * R) + grp * R;

  // Weight loads, unconditional from clamped addresses: a row past n reads
  // row n-1 and is not stored; a unit past U reads unit U-1 and meets zero
  // activations and zero B in LDS, so it adds exactly 0.
  const uint32_t t = li & 3u;
  const uint8_t *wrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    wrow[r] = w + (uint64_t)min(row_base + r, n - 1u) * nsb * 144u + 16u + 32u * t;
  auto load_unit = [&](uint32_t it, UnitLoads (&L)[R]) {
    const uint32_t sb = min(ub + li + G * it, U - 1u) >> 2;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint8_t *p = wrow[r] + sb * 144u;
      L[r].h = *reinterpret_cast<const uint4 *>(p - 16u - 32u * t);
      L[r].c0 = *reinterpret_cast<const uint4 *>(p);
      L[r].c1 = *reinterpret_cast<const uint4 *>(p + 16u);
    }
  };

  UnitLoads cur[R], nxt[R];
  // Activation prep: one item per (unit, sub-block): 32 values -> 16 pairs
  // and B.  The first item's activation loads go out before the first weight
  // loads: vector-memory counters retire in order, so the prep then waits for
  // the (L2-resident) activations only.
  auto prep = [&](uint32_t item, const uint4 (&v)[4]) {
    const uint32_t u = item >> 1, hs = item & 1u;
    uint32_t D[16] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w,
                      v[2].x, v[2].y, v[2].z, v[2].w, v[3].x, v[3].y, v[3].z, v[3].w};
    if (ub + u >= U) {
#pragma unroll
      for (int i = 0; i < 16; ++i) D[i] = 0u;
    }
    uint32_t p[16];
    act_pairs(D, p);
    act_pairs(D + 8, p + 8);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s = dot2(D[i], 0x3F803F80u, s);  // pairs times (1, 1)
    uint32_t *dst = smem + u * kUnitDw + 16u * hs;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint4 *>(dst + 4 * q) = make_uint4(p[4 * q], p[4 * q + 1], p[4 * q + 2], p[4 * q + 3]);
    smem[u * kUnitDw + 32u + hs] = __float_as_uint(-128.0f * s);
  };
  auto act_src = [&](uint32_t item) {
    // unit u = (super-block u / 4, chunk u % 4): values 64u .. 64u + 63
    return act + 64u * min(ub + (item >> 1), U - 1u) + 32u * (item & 1u);
  };
  auto load_act = [&](uint32_t item, uint4 (&v)[4]) {
    const uint4 *src = reinterpret_cast<const uint4 *>(act_src(item));
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = src[q];
  };
  // Lane-fixed positions of the two sub-blocks' 6-bit fields (j = 2t, 2t+1).
  // t < 2:  sc_j = S[j] & 63, m_j = S[j+4] & 63            (header words y, z)
  // t >= 2: sc_j = (S[j+4] & 15) | (S[j-4] >> 6) << 4,
  //         m_j  = (S[j+4] >> 4) | (S[j] >> 6) << 4         (words w, y, z)
  // With both cases written as bfe(low word, off, width) | bfe(word, off2,
  // width2) << 4 (width 0 extracts 0), every lane runs the same code.
  const bool hi_t = t >= 2u;
  const uint32_t sh = 16u * (t & 1u);
  const uint32_t wl = hi_t ? 4u : 6u, wh = hi_t ? 2u : 0u, om = hi_t ? 4u : 0u;
  const uint32_t mask = vconst(0x000F000Fu), magic = vconst(kMagic128);

  float acc_out[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc_out[r] = 0.0f;

  auto compute = [&](uint32_t it, const UnitLoads (&L)[R]) {
    const uint32_t u = li + G * it;
    const uint32_t *src = smem + u * kUnitDw;
    uint32_t P[32];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint4 v = *reinterpret_cast<const uint4 *>(src + 4 * q);
      P[4 * q] = v.x; P[4 * q + 1] = v.y; P[4 * q + 2] = v.z; P[4 * q + 3] = v.w;
    }
    const uint2 bb = *reinterpret_cast<const uint2 *>(src + 32);
    const float b_lo = __uint_as_float(bb.x), b_hi = __uint_as_float(bb.y);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t words[8] = {L[r].c0.x, L[r].c0.y, L[r].c0.z, L[r].c0.w,
                                 L[r].c1.x, L[r].c1.y, L[r].c1.z, L[r].c1.w};
      float a_lo = b_lo, a_hi = b_hi;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t x = words[i];
        a_lo = dot2(and_or(x, mask, magic), P[2 * i], a_lo);
        a_lo = dot2(and_or(x >> 8, mask, magic), P[2 * i + 1], a_lo);
        a_hi = dot2(and_or(x >> 4, mask, magic), P[16 + 2 * i], a_hi);
        a_hi = dot2(and_or(x >> 12, mask, magic), P[16 + 2 * i + 1], a_hi);
      }
      const uint4 h = L[r].h;
      const uint32_t ys = hi_t ? h.w : h.y, zs = hi_t ? h.w : h.z;
      const uint32_t sc_lo = __builtin_amdgcn_ubfe(ys, sh, wl) | (__builtin_amdgcn_ubfe(h.y, sh + 6u, wh) << 4);
      const uint32_t sc_hi = __builtin_amdgcn_ubfe(ys, sh + 8u, wl) | (__builtin_amdgcn_ubfe(h.y, sh + 14u, wh) << 4);
      const uint32_t m_lo = __builtin_amdgcn_ubfe(zs, sh + om, wl) | (__builtin_amdgcn_ubfe(h.z, sh + 6u, wh) << 4);
      const uint32_t m_hi = __builtin_amdgcn_ubfe(zs, sh + 8u + om, wl) | (__builtin_amdgcn_ubfe(h.z, sh + 14u, wh) << 4);
      const float d = f16_bits_to_f32(h.x & 0xFFFFu), dmin = f16_bits_to_f32(h.x >> 16);
      const float sdot = fmaf((float)sc_hi, a_hi, (float)sc_lo * a_lo);
      const float smin = fmaf((float)m_hi, b_hi, (float)m_lo * b_lo);
      acc_out[r] = fmaf(d, sdot, acc_out[r]);
      acc_out[r] = fmaf(dmin * 0.0078125f, smin, acc_out[r]);
    }
  };

  // The activation vector is staged chunk by chunk (one chunk for k <= 65536).
  for (;;) {
    const uint32_t Uc = kChunked ? min(U - ub, kChunkUnits) : U;
    const uint32_t iters = (Uc + G - 1) / G, Upad = iters * G;
    const uint32_t items = 2u * Upad;
    if (kChunked && ub > 0) __syncthreads();  // every lane is done with the previous chunk's LDS
    {
      const uint32_t first = min(tid, items - 1u);
      uint4 v[4];
      load_act(first, v);
      load_unit(0, cur);
      // lanes past the last item redo it: same values to the same LDS words
      prep(first, v);
    }
    for (uint32_t item = tid + kThreads; item < items; item += kThreads) {
      uint4 v[4];
      load_act(item, v);
      prep(item, v);
    }
    __syncthreads();

    // Two register sets alternate (unrolled by two, so nothing is copied); the
    // last one or two units are peeled so that every prefetch is unconditional.
    // The scheduling barriers keep each prefetch above the wait for the unit
    // being computed (left alone, the scheduler sinks the loads below it and
    // only one unit per lane is ever in flight).
    uint32_t it = 0;
    for (; it + 2 < iters; it += 2) {
      load_unit(it + 1, nxt);
      __builtin_amdgcn_sched_barrier(0);
      compute(it, cur);
      load_unit(it + 2, cur);
      __builtin_amdgcn_sched_barrier(0);
      compute(it + 1, nxt);
    }
    if (it + 1 < iters) {
      load_unit(it + 1, nxt);
      __builtin_amdgcn_sched_barrier(0);
      compute(it, cur);
      compute(it + 1, nxt);
    } else {
      compute(it, cur);
    }
    if (!kChunked) break;
    ub += kChunkUnits;
    if (ub >= U) break;
  }

  static_assert(G == 16 || G == 32, "row sums over 16 or 32 lanes");
#pragma unroll
  for (int r = 0; r < R; ++r) acc_out[r] = G == 16 ? row16_sum(acc_out[r]) : half_wave_sum(acc_out[r]);
  if (li == G - 1u) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t row = row_base + r;
      if (row < n) out[row] = (uint16_t)f32_to_bf16_rne(acc_out[r]);
    }
  }
}

template <int G, int R, bool kChunked>
hipError_t launch_g(const void *act, const void *w, void *out, uint32_t n, uint32_t k, hipStream_t s) {
  const uint32_t U = (k >> 8) * 4u, Uc = U < kChunkUnits ? U : kChunkUnits;
  const size_t lds = (size_t)((Uc + G - 1) / G * G) * kUnitDw * 4u;
  if (lds > 65536) {
    const hipError_t attr_err = ensure_dynamic_lds(
        reinterpret_cast<const void *>(q4k_gemv1_kernel<G, R, kChunked>), (int)((size_t)kChunkUnits * kUnitDw * 4u));
    if (attr_err != hipSuccess) return attr_err;
  }
  constexpr uint32_t rows_per_block = kThreads / G * R;
  const uint32_t blocks = (n + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL((q4k_gemv1_kernel<G, R, kChunked>), dim3(blocks), dim3(kThreads), lds, s,
                     static_cast<const uint16_t *>(act), static_cast<const uint8_t *>(w),
                     static_cast<uint16_t *>(out), n, k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_q4k_gemv(const void *act, const void *w, void *out, uint32_t n, uint32_t k,
                           hipStream_t s) {
  // Half-wave groups, one row per lane: measured on the FFN shapes against
  // 16-lane groups and two rows per lane (gate [17408, 5120] 11.3 us vs
  // 11.6 / 13.3 us; down [5120, 17408] 12.9 us vs 13.8 / 14.0 us): more
  // workgroups of fewer rows balance better over the compute units, and the
  // per-instruction footprint of one row per lane is more compact.
  if (k > 256u * kChunkUnits / 4u) return launch_g<32, 1, true>(act, w, out, n, k, s);
  return launch_g<32, 1, false>(act, w, out, n, k, s);
}

}  // namespace bqmm

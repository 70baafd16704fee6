/*
 * bqmm -- packed low-bit weight-quantized matmul for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every entry point takes plain pointers and sizes; device pointers
 * unless stated otherwise.  `stream` is a hipStream_t passed as void*; NULL
 * means the legacy default stream.  Every call enqueues its kernels on that
 * stream and returns without synchronizing: errors raised while the kernels
 * run surface at the caller's next synchronization.  No call allocates or
 * frees device memory or synchronizes; all buffers belong to the caller (the
 * reference dispatcher takes its scratch and q8_1 buffers from its caller
 * rather than allocating them: page layers/qwen3_ssm/init_q2.rs, fn
 * qkvz_q2_prefill_gemm).
 *
 * Errors are values, never aborts (the reference returns an error carrying a
 * message when a kernel or weight is missing: page
 * layers/dense_ffn_decode_batch.rs, fn forward_km_q2).  Every argument is
 * checked before any HIP call, so a rejected call touches no device state.
 * The message of the last failure on the calling thread is bq_last_error().
 *
 * Byte layouts (all little-endian; fp16 = IEEE binary16; bf16 = bfloat16):
 *
 *   q8_1 activations for [m][k], kpad = ceil(k/256)*256:
 *     codes plane, int8 [m][kpad] at byte 0; then the (d, s) plane: for row r
 *     and 32-value block b, fp16 d at byte m*kpad + 4*(r*kpad/32 + b) and
 *     fp16 s at +2.  d = fp16(amax/127) (binary32 division), q =
 *     clamp(roundf(x/d), -127, 127) using the stored d (binary32 division,
 *     ties away from zero), s = fp16(d * sum q); padding values are zero.
 *     Total q8_1_act_bytes(m, k) = 1.125*m*kpad bytes.
 *
 *   Q2_0 weight [n][k], group G (G = 128 for the matmul kernels):
 *     codes plane, n*k/4 bytes at byte 0: row r, group g occupies bytes
 *     [r*k/4 + g*G/4, +G/4); byte t of a group holds the 2-bit codes of
 *     k-offsets t + j*G/4 in bits [2j, 2j+1], j = 0..3.  Then the scale
 *     plane: fp16 d[r][g] at byte n*k/4 + 2*(r*k/G + g).  Weight value
 *     w = d*(c - 2), c in {0,1,2,3}.  Total q2_0_weight_bytes(n, k, G).
 *
 *   Q4_K weight [n][k]: row-major [n][k/256] super-blocks of 144 bytes:
 *     fp16 d (bytes 0-1), fp16 dmin (2-3), twelve bytes S of packed 6-bit
 *     sub-scales/mins (4-15), 128 bytes of 4-bit codes (16-143).  Sub-block
 *     j (32 weights): j < 4: sc = S[j] & 63, m = S[j+4] & 63; j >= 4:
 *     sc = (S[j+4] & 15) | ((S[j-4] >> 6) << 4), m = (S[j+4] >> 4) | ((S[j] >> 6) << 4).
 *     Byte 16 + 32t + i holds weight 64t+i (low nibble) and 64t+32+i (high
 *     nibble).  w = d*sc_j*q - dmin*m_j.  256 weights in 144 bytes as on page
 *     layers/ops/q4k_mmq.rs (consts QK_K, Q4K_BLOCK_BYTES).
 *
 * Alignment: weight, activation and q8_1 pointers must be 16-byte aligned
 * (BQ_EALIGN otherwise); bf16 row lengths used by vector loads are noted per
 * call.  Inputs and outputs must not overlap unless a call says so; every
 * call checks the byte ranges its shapes give and returns BQ_EINVAL when an
 * output range shares a byte with an input range.
 *
 * Size limits (BQ_EINVAL beyond them): k <= 2^30 and output rows n <= 2^31
 * for every call; the MMQs take m <= 65535*128 and the dense GEMM n <=
 * 65535*128 (tile counts in the second grid dimension); the Q4_K weight
 * quantizer takes n*k/256 super-blocks below 2^36 (one grid dimension).
 *
 * Only a gfx950 code object is built; on other devices calls fail with
 * BQ_EHIP.  The library keeps no mutable state besides the per-thread error
 * message and two lock-protected per-device records: the kernels whose
 * dynamic-LDS limit has been raised, and the compute-unit count (the MMQ and
 * the dense GEMM choose their tile shape from it; results do not depend on
 * the choice).  Calls from different threads are independent.
 */
#ifndef BQMM_H
#define BQMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define BQ_OK 0
#define BQ_EINVAL (-1)       /* null pointer, zero size, shape rule broken, overflow */
#define BQ_EUNSUPPORTED (-2) /* valid in principle but not provided (group, m > 8) */
#define BQ_EALIGN (-3)       /* pointer not 16-byte aligned */
#define BQ_EHIP (-4)         /* a HIP launch failed; the HIP message is in bq_last_error() */

/* Message of the last failing call on this thread ("" if none).  Host; the
 * string stays valid until the next call on the same thread. */
const char *bq_last_error(void);
/* Fixed description of a status code.  Host. */
const char *bq_status_string(int status);

/* ---- sizes (host) ------------------------------------------------------- */

/* Bytes of the q8_1 form of [m][k]: 1.125*m*kpad, kpad = ceil(k/256)*256.
 * The reference sizes its q8_1 scratch with k rounded up to 256 (page
 * layers/ops/q4k_mmq.rs, fn q8_1_scratch_bytes); its 4 bytes per value plus
 * 1 MiB over-allocates this exact size and may still be passed.  0 on overflow. */
uint64_t q8_1_act_bytes(uint32_t m, uint32_t k);

/* Bytes of a Q2_0 weight [n][k] with group `group`: n*k/4 + 2*n*k/group.
 * 0 if k % group != 0, group % 32 != 0 or on overflow. */
uint64_t q2_0_weight_bytes(uint32_t n, uint32_t k, uint32_t group);

/* Bytes of a Q4_K weight [n][k]: n*(k/256)*144 (page layers/ops/q4k_mmq.rs,
 * fn q4k_weight_bytes).  0 if k % 256 != 0 or on overflow. */
uint64_t q4k_weight_bytes(uint32_t n, uint32_t k);

/* ---- the hot path -------------------------------------------------------- */

/* bf16 activations [m][k] (row-major, contiguous) -> q8_1 in out_q8
 * (q8_1_act_bytes(m, k) bytes, layout above).
 * [page layers/ops/q4k_mmq.rs, fn quantize_act_q8_1: bf16 in, q8_1 out, k
 *  padded to 256.]  m >= 1, k >= 1.  act_bf16 and out_q8 16-byte aligned. */
int quantize_act_q8_1(const void *act_bf16, void *out_q8, uint32_t m, uint32_t k, void *stream);

/* The FFN hidden activation quantized straight from its producer:
 *   out_q8 = q8_1 of h,  h[i][j] = bf16_rne(silu(gate[i][j]) * up[i][j]),
 * i.e. silu_mul_bf16 followed by quantize_act_q8_1, without writing h; the
 * result equals those two calls bit for bit (same binary32 silu, same rule).
 * [page layers/dense_ffn_decode_batch.rs, fn forward_km_q2: silu_mul
 *  produces the down projection's input; page layers/ops/q4k_mmq.rs: each
 *  prefill quantizes its activations to q8_1.]
 * gate, up: [m][k] bf16; out_q8 holds q8_1_act_bytes(m, k) bytes.  m, k >= 1. */
int silu_mul_quantize_q8_1(const void *gate_bf16, const void *up_bf16, void *out_q8,
                           uint32_t m, uint32_t k, void *stream);

/* Q2_0 MMQ: out[m][n] (bf16, row-major, row stride n) =
 *   sum_k deq(act_q8)[m][k] * deq(w_q2)[n][k],
 * on int8 matrix cores with exact int32 block dot products; the scales are
 * applied after them: each q8_1 block scale as an exact integer multiplier
 * within a band of binary16 exponents (rounded by at most 2^-10 relative at
 * a band's lowest exponent; a tile whose rows span more takes one pass per
 * band), each weight group scale with an fp32 fma.
 * [page layers/qwen3_ssm/init_q2.rs, fn qkvz_q2_prefill_gemm:
 *  out[m, n] = input[m, k] @ W^T via quantize_act_q8_1 then q2_0_mmq_gemm,
 *  group 128 only.]
 * act_q8: q8_1 of [m][k]; w_q2: Q2_0 [n][k] with group 128.  k % 128 == 0,
 * m, n >= 1 (any n: tails handled inside). */
int q2_0_mmq_gemm(const void *act_q8, const void *w_q2, void *out_bf16,
                  uint32_t m, uint32_t n, uint32_t k, void *stream);

/* The MMQ GEMMs with an output row stride: out row i starts at out_bf16 +
 * i*ldc (ldc >= n, elements); the ldc - n columns between rows are not
 * written.  Lets a projection write straight into a column range of a wider
 * buffer (pass the range's first element as out_bf16), e.g. the segments of
 * the deinterleaved qkvz buffer.  [page layers/qwen3_ssm/init_q2.rs, fn
 *  qkvz_q2_prefill_gemm / fn set_packed_q2_qkvz: the packed qkvz projection
 *  and the buffer it fills; page layers/ops/q4k_mmq.rs, fn q4k_mmq_gemm.]
 * Constraints as for q2_0_mmq_gemm / q4k_mmq_gemm; out_bf16 16-byte aligned. */
int q2_0_mmq_gemm_ldc(const void *act_q8, const void *w_q2, void *out_bf16,
                      uint32_t m, uint32_t n, uint32_t k, uint32_t ldc, void *stream);
int q4k_mmq_gemm_ldc(const void *act_q8, const void *w_q4k, void *out_bf16,
                     uint32_t m, uint32_t n, uint32_t k, uint32_t ldc, void *stream);

/* Q2_0 decode GEMV, one row: out[n] (bf16) = sum_k act[k] * deq(w_q2)[n][k],
 * on the unquantized bf16 activation, fp32 accumulation.
 * [page layers/qwen3_ssm/init.rs, kernel q2_0_gemv_vec; page
 *  layers/qwen3_ssm/init_q2.rs, fn set_packed_q2_qkvz: decode runs the GEMV
 *  on the packed qkvz.]  Group 128; k % 128 == 0; n >= 1. */
int q2_0_gemv_vec(const void *act_bf16, const void *w_q2, void *out_bf16,
                  uint32_t n, uint32_t k, void *stream);

/* Q2_0 GEMV for m = 1..8 rows (small verify batches): act [m][k] bf16,
 * out [m][n] bf16.  [page layers/dense_ffn_decode_batch.rs, fn forward_km_q2:
 *  q2_0_gemv_vec_batchm(inp, w, out, m).]  m > 8 -> BQ_EUNSUPPORTED.
 * Group 128; k % 128 == 0.
 * Kernels: m = 1, 2 run on the vector ALU only (packed bf16 dot products, no
 * matrix cores).  From m = 3 on, where the per-code multiply-adds outweigh
 * the code unpacking, the products run on bf16 matrix cores
 * (v_mfma_f32_16x16x32_bf16, codes and activations exact in bf16, fp32
 * accumulation): a deliberate exception to keeping the GEMV a pure
 * bandwidth kernel, taken because it measured faster at these m.  Where the
 * matrix-core kernel's LDS (staged weight scales and 1 KB per wave for the
 * weight loads) would exceed 64 KB in the fused gate/up launch (k above
 * 37888), both calls use the vector kernel. */
int q2_0_gemv_vec_batchm(const void *act_bf16, const void *w_q2, void *out_bf16,
                         uint32_t m, uint32_t n, uint32_t k, void *stream);

/* Fused FFN gate/up GEMV with the SiLU-gated product, m = 1..8 rows:
 *   out[i][r] = bf16_rne(silu(g) * u),  g = bf16_rne(sum_k act[i][k] * deq(w_gate)[r][k]),
 *                                       u = bf16_rne(sum_k act[i][k] * deq(w_up)[r][k]),
 * i.e. q2_0_gemv_vec_batchm on both weights followed by silu_mul_bf16, in one
 * launch that reads the activations once.  For m = 2..8 the result equals
 * that three-call chain bit for bit (same kernels, same summation order).
 * [page layers/dense_ffn_decode_batch.rs, fn forward_km_q2: gate and up
 *  GEMVs, then silu_mul into the gate buffer.]
 * act [m][k] bf16; w_gate, w_up: Q2_0 [n][k] group 128; out [m][n] bf16 and
 * must not overlap act or either weight.  k % 128 == 0, n >= 1,
 * m > 8 -> BQ_EUNSUPPORTED. */
int q2_0_gemv_gate_up_silu(const void *act_bf16, const void *w_gate_q2, const void *w_up_q2,
                           void *out_bf16, uint32_t m, uint32_t n, uint32_t k, void *stream);

/* Q2_0 weight -> bf16 [n][k]: bf16_rne(d*(c - 2)) (exact product, one
 * rounding).  [page layers/qwen3_ssm/init_q2.rs, fn qkvz_q2_prefill_gemm,
 *  fallback: dequant_q2_0_gn_to_bf16(w, scratch, n, k, group).]
 * group % 32 == 0 and k % group == 0. */
int dequant_q2_0_to_bf16(const void *w_q2, void *out_bf16, uint32_t n, uint32_t k,
                         uint32_t group, void *stream);

/* Dense bf16 GEMM: out[m][n] (bf16) = sum_k a[m][k] * w[n][k], fp32
 * accumulation.  [page layers/qwen3_ssm/init_q2.rs, fn qkvz_q2_prefill_gemm,
 *  fallback: dense_gemm_bf16_pipelined on the original bf16 input.]
 * k % 64 == 0; m, n >= 1. */
int dense_gemm_bf16(const void *a_bf16, const void *w_bf16, void *out_bf16,
                    uint32_t m, uint32_t n, uint32_t k, void *stream);

/* Prefill dispatcher.  With use_mmq != 0 and group == 128: quantize act_bf16
 * into act_q8 (q8_1_act_bytes(m, k) bytes) and run q2_0_mmq_gemm.  Otherwise
 * dequantize the weight into scratch_bf16 (n*k*2 bytes) and run
 * dense_gemm_bf16 on the original bf16 input.  Both on `stream`.
 * [page layers/qwen3_ssm/init_q2.rs, fn qkvz_q2_prefill_gemm.]  The buffer
 * the chosen branch does not use may be NULL. */
int q2_0_prefill_gemm(const void *act_bf16, const void *w_q2, void *out_bf16,
                      void *scratch_bf16, void *act_q8, uint32_t m, uint32_t n, uint32_t k,
                      uint32_t group, int use_mmq, void *stream);

/* The prefill dispatcher for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same branches, kernels and results as q2_0_prefill_gemm, with the branch's
 * workspace (the q8_1 buffer, or the bf16 dequant buffer) taken from a
 * 64 MiB device array the library holds on every GPU it runs on, from the
 * code object's load until the process ends.  The call itself allocates
 * nothing.  Limits: the MMQ branch needs q8_1_act_bytes(m, k) <= 64 MiB
 * (m * kpad <= 59,652,323, e.g. m = 4096 at k = 14336), the dequant branch
 * n * k * 2 <= 64 MiB (n * k <= 33,554,432); larger shapes return
 * BQ_EUNSUPPORTED before any HIP call.  Every call on a GPU shares that
 * GPU's array: calls that overlap in time on one GPU (two streams, or two
 * host threads) race on it and must be ordered by the caller.  The array's
 * contents are not cleared; each branch writes every byte it reads. */
int q2_0_prefill_gemm_noalloc(const void *act_bf16, const void *w_q2, void *out_bf16,
                              uint32_t m, uint32_t n, uint32_t k, uint32_t group, int use_mmq,
                              void *stream);

/* Q4_K MMQ: out[m][n] (bf16) = sum_k deq(act_q8)[m][k] * deq_q4k(w)[n][k],
 * on fp16 matrix cores: the weight operand q4 * sc_j is exact, the
 * activation operand is q * da * 2^-e rounded once to binary16 (relative
 * error at most 2^-11; e per activation row, from its largest da; a block
 * more than 2^22 below that largest loses one bit of its scale per binade,
 * and beyond about 2^33 contributes nothing), the min term from the exact
 * m_j and the stored q8_1 sums times 2^-(e + 6), d and dmin applied in fp32
 * once per super-block and 2^e once per output.
 * [page layers/ops/q4k_mmq.rs, fn q4k_mmq_gemm: C[m, n] = A[m, k] x W[n, k],
 *  A in q8_1, W in block_q4_K, BF16 store; any n.]  k % 256 == 0. */
int q4k_mmq_gemm(const void *act_q8, const void *w_q4k, void *out_bf16,
                 uint32_t m, uint32_t n, uint32_t k, void *stream);

/* Q4_K decode GEMV, one row: out[n] (bf16) = sum_k act[k] * deq_q4k(w)[n][k],
 * on the unquantized bf16 activation, fp32 accumulation; deq_q4k as for
 * q4k_mmq_gemm (w = d * sc_j * q - dmin * m_j per 32-weight sub-block).
 * [page layers/ops/q4k_mmq.rs: block_q4_K and fn q4k_mmq_gemm, C = A x W^T;
 *  the bf16-input decode form follows the Q2_0 decode GEMV, page
 *  layers/qwen3_ssm/init.rs, q2_0_gemv_vec.]
 * act_bf16: [k]; w_q4k: [n][k/256] blocks of 144 bytes; out_bf16: [n].
 * k % 256 == 0 (the activation vector is staged in LDS 65536 values at a
 * time); n >= 1. */
int q4k_gemv_vec(const void *act_bf16, const void *w_q4k, void *out_bf16,
                 uint32_t n, uint32_t k, void *stream);

/* Q4_K weight quantization: out_q4k ([n][k/256] blocks of 144 bytes,
 * q4k_weight_bytes(n, k)) from w_bf16 ([n][k] bf16, row-major).
 * [page layers/ops/q4k_mmq.rs, fn quantize_weight_q4k: bf16 [nrows,
 *  n_per_row] to block_q4_K, one 256-value block per thread.]  The page gives
 * no rule; the one implemented, bit-exact, in binary32 with IEEE division
 * and roundf (ties away from zero), per 32-value sub-block j:
 *   lo_j = min(+0, min x), hi_j = max(lo_j, max x),
 *   S_j = (hi_j - lo_j) / 15, M_j = 0 - lo_j,
 *   d = fp16_rne(max_j S_j / 63), dmin = fp16_rne(max_j M_j / 63),
 *   sc_j = d > 0 ? min(63, roundf(S_j / d)) : 0 (m_j likewise from M_j, dmin),
 *   q = clamp(roundf((x + dmin*m_j) / (d*sc_j)), 0, 15), 0 if d*sc_j == 0.
 * Supported range: finite inputs with max S_j / 63 and max M_j / 63 within
 * binary16 (|x| below about 1.5e7); outside it the bytes are unspecified.
 * k % 256 == 0; n >= 1; both buffers 16-byte aligned. */
int quantize_weight_q4k(const void *w_bf16, void *out_q4k, uint32_t n, uint32_t k,
                        void *stream);

/* out[i] = bf16_rne(silu(gate[i]) * up[i]) for i < count, silu(g) =
 * g/(1+exp(-g)) in fp32 with the hardware exp2 and reciprocal: within one bf16
 * step of the exact value for gate >= -87; below about -87.3 the result is +-0
 * (the exact value is under 1e-35 * |up| there).  out == gate is allowed (in
 * place).
 * [page layers/dense_ffn_decode_batch.rs, fn forward_km_q2: silu_mul over
 *  m * intermediate elements with the output over the gate buffer.] */
int silu_mul_bf16(const void *gate, const void *up, void *out, uint64_t count, void *stream);

/* ---- test hooks: integer block dot products ---------------------------- */

/* Runs the MMQ kernel's own unpack and matrix-core path over the window
 * rows [m0, m0+mt) x columns [n0, n0+nt) and writes, instead of the scaled
 * output, the int32 dot product of every 32-block:
 *   out[(i*nt + j)*(k/32) + b] = sum_{t<32} (c - 2) * q     (Q2_0)
 *   out[(i*nt + j)*(k/32) + b] = sum_{t<32} q4 * q          (Q4_K)
 * for row m0+i, column n0+j, block b.  out holds mt*nt*(k/32) int32.
 * Constraints as for the matching GEMM; mt, nt >= 1; the window must lie
 * inside [0, m) x [0, n). */
int q2_0_mmq_blockdots(const void *act_q8, const void *w_q2, int32_t *out,
                       uint32_t m0, uint32_t mt, uint32_t n0, uint32_t nt,
                       uint32_t m, uint32_t n, uint32_t k, void *stream);
int q4k_mmq_blockdots(const void *act_q8, const void *w_q4k, int32_t *out,
                      uint32_t m0, uint32_t mt, uint32_t n0, uint32_t nt,
                      uint32_t m, uint32_t n, uint32_t k, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BQMM_H */

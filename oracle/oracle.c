/*
 * CPU oracle for the packed low-bit weight-quantized matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Plain, slow, single-threaded C11 (-O2, no
 * fast-math, no SIMD intrinsics, no threads).  Nothing in the product path
 * may link, load or call this file: only tests/, the smoke check in
 * __graft_entry__.py and the cpu_baseline leg of bench.py use it.  It shares
 * no source, header, table or helper with the HIP library.  Each byte layout
 * is restated next to the routine that reads it.
 *
 * Every routine states the passage of the reference pages it follows.  The
 * pages are rustdoc source views of the crate `metrale_model_layers`; they are
 * cited as  [page <file>, <item>].  The pages give launch shapes and names,
 * not bit layouts or rounding rules; where they are silent the reading taken
 * is stated next to the code.
 *
 * Floating point: every result that the method reaches exactly (dequantized
 * values, products, dot products) is formed in fp64, which is exact for all
 * of them except the final sums.  Where floating point decides an integer --
 * the q8_1 code of an activation, the sub-scales and codes of the Q4_K weight
 * quantizer -- it is taken in fp32 with IEEE division and C roundf, the
 * precision the kernels use.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

/* ------------------------------------------------------------------------ */
/* Scalar conversions (IEEE binary16 / bfloat16 <-> binary32 / binary64).   */
/* ------------------------------------------------------------------------ */

float oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t e = (h >> 10) & 0x1Fu;
    uint32_t f = h & 0x3FFu;
    float v;
    if (e == 0) {
        v = ldexpf((float)f, -24); /* zero or subnormal: f * 2^-24 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexpf((float)(f | 0x400u), (int)e - 25);
    }
    uint32_t bits;
    memcpy(&bits, &v, 4);
    bits |= sign;
    memcpy(&v, &bits, 4);
    return v;
}

/* binary32 -> binary16, round to nearest, ties to even. */
uint16_t oracle_f32_to_f16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return (uint16_t)(sign | 0x7E00u); /* NaN */
    if (a >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u); /* >= 65520 -> inf */
    int e = (int)(a >> 23);            /* biased binary32 exponent */
    uint32_t sig = (a & 0x7FFFFFu) | (e ? 0x800000u : 0u);
    if (e == 0) e = 1;                 /* binary32 subnormal */
    /* value = sig * 2^(e-150); binary16 unit in the last place is
     * 2^(max(e-127,-14) - 10).  Shift sig so that one unit is 1. */
    int ulp_exp = (e - 127 < -14 ? -14 : e - 127) - 10;
    int shift = ulp_exp - (e - 150); /* >= 13 */
    if (shift >= 32) return sign; /* below a quarter of the smallest subnormal */
    uint32_t q = sig >> shift;
    uint32_t rem = sig & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) q++;
    /* q counts units of 2^ulp_exp; rebuild the binary16 bit pattern */
    uint32_t h;
    if (ulp_exp == -24) {
        h = q;                   /* subnormal; q == 0x400 is the smallest normal */
    } else {
        /* q in [0x400, 0x800]; 0x800 carries into the exponent */
        uint32_t be = (uint32_t)(ulp_exp + 10 + 15);
        h = (be << 10) + (q - 0x400u);
    }
    return (uint16_t)(sign | h);
}

double oracle_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* binary64 -> bfloat16, round to nearest, ties to even, in one rounding. */
uint16_t oracle_f64_to_bf16(double x)
{
    if (isnan(x)) return 0x7FC0u;
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(x);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                /* a = fr * 2^e, fr in [0.5, 1) */
    int ulp_exp = e - 8;         /* 8 significant bits */
    if (ulp_exp < -133) ulp_exp = -133; /* bfloat16 subnormal unit 2^-133 */
    double q = nearbyint(ldexp(a, -ulp_exp)); /* default mode: ties to even */
    double r = ldexp(q, ulp_exp);
    if (r > 3.3895313892515355e+38) return (uint16_t)(sign | 0x7F80u); /* > max bf16 */
    float rf = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &rf, 4);
    return (uint16_t)(sign | (u >> 16));
}

/* ------------------------------------------------------------------------ */
/* q8_1 activations                                                          */
/* ------------------------------------------------------------------------ */

/* k padded to a whole number of 256-value super-blocks.
 * [page layers/ops/q4k_mmq.rs, fn quantize_act_q8_1 and fn q8_1_scratch_bytes:
 *  the activation row is padded to a multiple of QK_K = 256.] */
uint64_t oracle_q8_1_kpad(uint32_t k)
{
    return ((uint64_t)k + 255u) / 256u * 256u;
}

uint64_t oracle_q8_1_bytes(uint32_t m, uint32_t k)
{
    uint64_t kp = oracle_q8_1_kpad(k);
    return (uint64_t)m * kp + (uint64_t)m * (kp / 32u) * 4u;
}

/* Quantize bf16 activations [m][k] to q8_1.
 * [page layers/ops/q4k_mmq.rs, fn quantize_act_q8_1: bf16 in, q8_1 out, row
 *  padded to 256; blocks of 32 int8 values, each with a scale d and a sum s.]
 * Readings (the page names the encoding but prints no rule):
 *  d = fp16_rne(amax / 127) in fp32; codes from the stored fp16 d with IEEE
 *  division and roundf (ties away from zero), clamped to [-127, 127];
 *  s = fp16_rne(d * sum(q)); padding values are 0.
 * Layout: codes plane int8 [m][kpad], then the (d, s) plane: for row r and
 *  block b the fp16 pair sits at byte m*kpad + 4*(r*kpad/32 + b).
 * Returns the number of blocks whose amax exceeds 2047 or is not finite (the
 * supported range: there s or d may overflow binary16); 0 otherwise. */
int64_t oracle_quantize_act_q8_1(const uint16_t *act, uint8_t *out, uint32_t m, uint32_t k)
{
    uint64_t kp = oracle_q8_1_kpad(k);
    uint64_t nb = kp / 32u;
    uint8_t *ds = out + (uint64_t)m * kp;
    int64_t flagged = 0;
    for (uint64_t r = 0; r < m; ++r) {
        for (uint64_t b = 0; b < nb; ++b) {
            float x[32];
            float amax = 0.0f;
            int finite = 1;
            for (int i = 0; i < 32; ++i) {
                uint64_t kk = b * 32u + (uint64_t)i;
                x[i] = kk < k ? (float)oracle_bf16_to_f64(act[r * k + kk]) : 0.0f;
                if (!isfinite(x[i])) finite = 0;
                float ax = fabsf(x[i]);
                if (ax > amax) amax = ax;
            }
            if (!finite || amax > 2047.0f) flagged++;
            uint16_t dh = oracle_f32_to_f16(amax / 127.0f);
            float d = oracle_f16_to_f32(dh);
            int32_t sum = 0;
            for (int i = 0; i < 32; ++i) {
                int32_t q = 0;
                if (d != 0.0f) {
                    float t = roundf(x[i] / d);
                    if (t > 127.0f) t = 127.0f;
                    if (t < -127.0f) t = -127.0f;
                    q = t == t ? (int32_t)t : 0; /* NaN (a flagged block): 0, not undefined */
                }
                out[r * kp + b * 32u + (uint64_t)i] = (uint8_t)(int8_t)q;
                sum += q;
            }
            uint16_t sh = oracle_f32_to_f16(d * (float)sum);
            uint8_t *p = ds + 4u * (r * nb + b);
            p[0] = (uint8_t)(dh & 0xFFu);
            p[1] = (uint8_t)(dh >> 8);
            p[2] = (uint8_t)(sh & 0xFFu);
            p[3] = (uint8_t)(sh >> 8);
        }
    }
    return flagged;
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Dequantized q8_1 activations, fp64 [m][kpad]: value = float(d) * q. */
void oracle_dequant_q8_1(const uint8_t *q8, double *out, uint32_t m, uint32_t k)
{
    uint64_t kp = oracle_q8_1_kpad(k);
    uint64_t nb = kp / 32u;
    const uint8_t *ds = q8 + (uint64_t)m * kp;
    for (uint64_t r = 0; r < m; ++r)
        for (uint64_t b = 0; b < nb; ++b) {
            double d = (double)oracle_f16_to_f32(rd16(ds + 4u * (r * nb + b)));
            for (int i = 0; i < 32; ++i) {
                int8_t q = (int8_t)q8[r * kp + b * 32u + (uint64_t)i];
                out[r * kp + b * 32u + (uint64_t)i] = d * (double)q;
            }
        }
}

/* ------------------------------------------------------------------------ */
/* Q2_0 weights                                                              */
/* ------------------------------------------------------------------------ */

uint64_t oracle_q2_0_bytes(uint32_t n, uint32_t k, uint32_t group)
{
    return (uint64_t)n * k / 4u + 2u * ((uint64_t)n * (k / group));
}

/* The 2-bit code of weight (r, kk).
 * [page layers/qwen3_ssm/init_q2.rs, fn set_packed_q2_qkvz and
 *  fn qkvz_q2_prefill_gemm: one packed pointer carries codes and per-group
 *  scales; group size is a property of the weight.]
 * Adopted layout: codes plane first, n*k/4 bytes; row r, group g occupies
 * bytes [r*k/4 + g*G/4, +G/4); byte t of a group holds the codes of k-offsets
 * t + j*G/4 in bits [2j, 2j+1], j = 0..3. */
static uint32_t q2_code(const uint8_t *w, uint32_t k, uint32_t group, uint64_t r, uint64_t kk)
{
    uint64_t g = kk / group;
    uint64_t off = kk % group;
    uint64_t quarter = group / 4u;
    uint64_t t = off % quarter;
    uint64_t j = off / quarter;
    uint8_t byte = w[r * (k / 4u) + g * quarter + t];
    return (byte >> (2u * j)) & 3u;
}

/* Scale plane after the codes: fp16 d[r][g] at n*k/4 + 2*(r*k/G + g). */
static double q2_scale(const uint8_t *w, uint32_t n, uint32_t k, uint32_t group, uint64_t r, uint64_t g)
{
    const uint8_t *sp = w + (uint64_t)n * k / 4u;
    return (double)oracle_f16_to_f32(rd16(sp + 2u * (r * (k / group) + g)));
}

/* Dequantized Q2_0 weight, fp64 [n][k]: w = float(d) * (c - 2). */
void oracle_q2_0_decode(const uint8_t *w, double *out, uint32_t n, uint32_t k, uint32_t group)
{
    for (uint64_t r = 0; r < n; ++r)
        for (uint64_t kk = 0; kk < k; ++kk) {
            double d = q2_scale(w, n, k, group, r, kk / group);
            out[r * k + kk] = d * ((double)q2_code(w, k, group, r, kk) - 2.0);
        }
}

/* Weight dequantized to bf16 [n][k]: bf16_rne(float(d) * (c - 2)).
 * [page layers/qwen3_ssm/init_q2.rs, fn qkvz_q2_prefill_gemm, fallback
 *  branch: dequant_q2_0_gn_to_bf16 writes the weight as BF16 into scratch.]
 * The product is exact, so this is one rounding of the exact value. */
void oracle_dequant_q2_0_to_bf16(const uint8_t *w, uint16_t *out, uint32_t n, uint32_t k, uint32_t group)
{
    for (uint64_t r = 0; r < n; ++r)
        for (uint64_t kk = 0; kk < k; ++kk) {
            double d = q2_scale(w, n, k, group, r, kk / group);
            out[r * k + kk] = oracle_f64_to_bf16(d * ((double)q2_code(w, k, group, r, kk) - 2.0));
        }
}

/* Integer dot product of q8_1 block b of activation row i with the signed
 * codes of weight row j: D[i][j][b] = sum over the block of (c - 2) * q.
 * This is the quantity an int8 matrix core accumulates per 32-block before
 * any scale is applied.  Group 128. */
void oracle_q2_0_blockdots(const uint8_t *q8, const uint8_t *w, int32_t *D,
                           uint32_t m, uint32_t n, uint32_t k)
{
    uint64_t kp = oracle_q8_1_kpad(k);
    uint64_t nb = k / 32u;
    for (uint64_t i = 0; i < m; ++i)
        for (uint64_t j = 0; j < n; ++j)
            for (uint64_t b = 0; b < nb; ++b) {
                int32_t acc = 0;
                for (uint64_t t = 0; t < 32; ++t) {
                    uint64_t kk = b * 32u + t;
                    int32_t c = (int32_t)q2_code(w, k, 128u, j, kk) - 2;
                    acc += c * (int32_t)(int8_t)q8[i * kp + kk];
                }
                D[(i * n + j) * nb + b] = acc;
            }
}

/* Q2_0 MMQ: R[i][j] = sum_k deq(a_q8)[i][k] * deq(W)[j][k], fp64.
 * [page layers/qwen3_ssm/init_q2.rs, fn qkvz_q2_prefill_gemm: out[m, n] =
 *  input[m, k] @ W^T through quantize_act_q8_1 then q2_0_mmq_gemm, group 128.]
 * Plain definition on the dequantized operands; one weight row is decoded at
 * a time. */
void oracle_q2_0_mmq(const uint8_t *q8, const uint8_t *w, double *R,
                     uint32_t m, uint32_t n, uint32_t k)
{
    uint64_t kp = oracle_q8_1_kpad(k);
    double *a = (double *)malloc(sizeof(double) * (uint64_t)m * kp);
    double *row = (double *)malloc(sizeof(double) * k);
    oracle_dequant_q8_1(q8, a, m, k);
    for (uint64_t j = 0; j < n; ++j) {
        for (uint64_t kk = 0; kk < k; ++kk)
            row[kk] = q2_scale(w, n, k, 128u, j, kk / 128u) *
                      ((double)q2_code(w, k, 128u, j, kk) - 2.0);
        for (uint64_t i = 0; i < m; ++i) {
            double s = 0.0;
            for (uint64_t kk = 0; kk < k; ++kk) s += a[i * kp + kk] * row[kk];
            R[i * n + j] = s;
        }
    }
    free(row);
    free(a);
}

/* Q2_0 GEMV on unquantized bf16 activations, m rows (m = 1 for decode).
 * [page layers/qwen3_ssm/init.rs, q2_0_gemv_vec lookup; page
 *  layers/dense_ffn_decode_batch.rs, fn forward_km_q2: q2_0_gemv_vec_batchm
 *  takes the bf16 activation buffer directly, no quantize step.]
 * R[i][j] = sum_k a_bf16[i][k] * float(d)(c - 2), fp64.  Group 128. */
void oracle_q2_0_gemv(const uint16_t *act, const uint8_t *w, double *R,
                      uint32_t m, uint32_t n, uint32_t k)
{
    double *a = (double *)malloc(sizeof(double) * (uint64_t)m * k);
    double *row = (double *)malloc(sizeof(double) * k);
    for (uint64_t i = 0; i < (uint64_t)m * k; ++i) a[i] = oracle_bf16_to_f64(act[i]);
    for (uint64_t j = 0; j < n; ++j) {
        for (uint64_t kk = 0; kk < k; ++kk)
            row[kk] = q2_scale(w, n, k, 128u, j, kk / 128u) *
                      ((double)q2_code(w, k, 128u, j, kk) - 2.0);
        for (uint64_t i = 0; i < m; ++i) {
            double s = 0.0;
            for (uint64_t kk = 0; kk < k; ++kk) s += a[i * k + kk] * row[kk];
            R[i * n + j] = s;
        }
    }
    free(row);
    free(a);
}

/* Dense GEMM on bf16 operands: R[i][j] = sum_k a[i][k] * w[j][k], fp64.
 * [page layers/qwen3_ssm/init_q2.rs, fn qkvz_q2_prefill_gemm, fallback:
 *  dense_gemm_bf16_pipelined / dense_gemm on the original bf16 input.] */
void oracle_dense_gemm_bf16(const uint16_t *a, const uint16_t *w, double *R,
                            uint32_t m, uint32_t n, uint32_t k)
{
    for (uint64_t i = 0; i < m; ++i)
        for (uint64_t j = 0; j < n; ++j) {
            double s = 0.0;
            for (uint64_t kk = 0; kk < k; ++kk)
                s += oracle_bf16_to_f64(a[i * k + kk]) * oracle_bf16_to_f64(w[j * k + kk]);
            R[i * n + j] = s;
        }
}

/* out = bf16_rne(silu(g) * u), silu(g) = g / (1 + exp(-g)), in fp64.
 * [page layers/dense_ffn_decode_batch.rs, fn forward_km_q2: silu_mul over
 *  m * intermediate elements, written in place over the gate buffer.] */
void oracle_silu_mul_bf16(const uint16_t *g, const uint16_t *u, uint16_t *out, uint64_t count)
{
    for (uint64_t i = 0; i < count; ++i) {
        double gv = oracle_bf16_to_f64(g[i]);
        double uv = oracle_bf16_to_f64(u[i]);
        out[i] = oracle_f64_to_bf16(gv / (1.0 + exp(-gv)) * uv);
    }
}

/* Round fp64 values to bf16 (RNE), for stage-wise chain comparisons. */
void oracle_round_bf16(const double *in, uint16_t *out, uint64_t count)
{
    for (uint64_t i = 0; i < count; ++i) out[i] = oracle_f64_to_bf16(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Q4_K weights                                                              */
/* ------------------------------------------------------------------------ */

/* [page layers/ops/q4k_mmq.rs, consts QK_K and Q4K_BLOCK_BYTES and
 *  fn q4k_weight_bytes: 256 weights per block_q4_K, 144 bytes each,
 *  nrows * (n_per_row / 256) * 144 bytes.] */
uint64_t oracle_q4k_bytes(uint32_t n, uint32_t k)
{
    return (uint64_t)n * (k / 256u) * 144u;
}

/* Sub-block scale and min of super-block `blk` (144 bytes), sub-block j.
 * Adopted layout: the public GGUF block_q4_K -- bytes 0-1 fp16 d, 2-3 fp16
 * dmin, 4-15 twelve bytes S of packed 6-bit scales and mins, 16-143 the
 * 4-bit codes.  For j < 4: sc = S[j] & 63, m = S[j+4] & 63; for j >= 4:
 * sc = (S[j+4] & 15) | ((S[j-4] >> 6) << 4), m = (S[j+4] >> 4) | ((S[j] >> 6) << 4). */
static void q4k_scale_min(const uint8_t *blk, int j, uint32_t *sc, uint32_t *mn)
{
    const uint8_t *S = blk + 4;
    if (j < 4) {
        *sc = S[j] & 63u;
        *mn = S[j + 4] & 63u;
    } else {
        *sc = (uint32_t)(S[j + 4] & 15u) | ((uint32_t)(S[j - 4] >> 6) << 4);
        *mn = (uint32_t)(S[j + 4] >> 4) | ((uint32_t)(S[j] >> 6) << 4);
    }
}

/* 4-bit code of weight e (0..255) of a super-block: in 64-weight chunk
 * t = e / 64, byte 16 + 32t + (e % 32) holds weight 64t + i in its low
 * nibble and weight 64t + 32 + i in its high nibble. */
static uint32_t q4k_code(const uint8_t *blk, uint32_t e)
{
    uint32_t t = e / 64u, within = e % 64u;
    uint8_t byte = blk[16u + 32u * t + (within % 32u)];
    return within < 32u ? (byte & 15u) : (uint32_t)(byte >> 4);
}

/* Dequantized Q4_K weight, fp64 [n][k]: w = d * sc_j * q - dmin * m_j. */
void oracle_q4k_decode(const uint8_t *w, double *out, uint32_t n, uint32_t k)
{
    uint64_t nsb = k / 256u;
    for (uint64_t r = 0; r < n; ++r)
        for (uint64_t s = 0; s < nsb; ++s) {
            const uint8_t *blk = w + (r * nsb + s) * 144u;
            double d = (double)oracle_f16_to_f32(rd16(blk));
            double dmin = (double)oracle_f16_to_f32(rd16(blk + 2));
            for (uint32_t e = 0; e < 256u; ++e) {
                uint32_t sc, mn;
                q4k_scale_min(blk, (int)(e / 32u), &sc, &mn);
                out[r * k + s * 256u + e] = d * (double)sc * (double)q4k_code(blk, e) - dmin * (double)mn;
            }
        }
}

/* D[i][j][b] = sum over 32-block b of q4 * q (unsigned 4-bit code times the
 * int8 activation code): the integer dot of one sub-block. */
void oracle_q4k_blockdots(const uint8_t *q8, const uint8_t *w, int32_t *D,
                          uint32_t m, uint32_t n, uint32_t k)
{
    uint64_t kp = oracle_q8_1_kpad(k);
    uint64_t nb = k / 32u, nsb = k / 256u;
    for (uint64_t i = 0; i < m; ++i)
        for (uint64_t j = 0; j < n; ++j)
            for (uint64_t b = 0; b < nb; ++b) {
                const uint8_t *blk = w + (j * nsb + b / 8u) * 144u;
                int32_t acc = 0;
                for (uint32_t t = 0; t < 32u; ++t) {
                    uint32_t e = (uint32_t)(b % 8u) * 32u + t;
                    acc += (int32_t)q4k_code(blk, e) * (int32_t)(int8_t)q8[i * kp + b * 32u + t];
                }
                D[(i * n + j) * nb + b] = acc;
            }
}

/* Q4_K MMQ: R[i][j] = sum_k deq(a_q8)[i][k] * deq_q4k(W)[j][k], fp64.
 * [page layers/ops/q4k_mmq.rs, fn q4k_mmq_gemm: C[m, n] = A[m, k] x W[n, k]
 *  with A in q8_1 and W in block_q4_K, BF16 store.]  Plain definition. */
void oracle_q4k_mmq(const uint8_t *q8, const uint8_t *w, double *R,
                    uint32_t m, uint32_t n, uint32_t k)
{
    uint64_t kp = oracle_q8_1_kpad(k);
    double *a = (double *)malloc(sizeof(double) * (uint64_t)m * kp);
    double *row = (double *)malloc(sizeof(double) * k);
    oracle_dequant_q8_1(q8, a, m, k);
    for (uint64_t j = 0; j < n; ++j) {
        oracle_q4k_decode(w + j * (k / 256u) * 144u, row, 1u, k);
        for (uint64_t i = 0; i < m; ++i) {
            double s = 0.0;
            for (uint64_t kk = 0; kk < k; ++kk) s += a[i * kp + kk] * row[kk];
            R[i * n + j] = s;
        }
    }
    free(row);
    free(a);
}

/* Q4_K GEMV on unquantized bf16 activations, m rows (m = 1 for decode):
 * R[i][j] = sum_k a_bf16[i][k] * deq_q4k(W)[j][k], fp64.
 * [page layers/ops/q4k_mmq.rs, fn q4k_mmq_gemm: C[m, n] = A[m, k] x W[n, k]
 *  with W in block_q4_K.]  The pages run Q4_K only through q8_1 and the MMQ;
 * the decode form taken here is the same product on the bf16 activations
 * with no quantize step, as the Q2_0 decode GEMV takes them
 * ([page layers/qwen3_ssm/init.rs, q2_0_gemv_vec]).  Plain definition. */
void oracle_q4k_gemv(const uint16_t *act, const uint8_t *w, double *R,
                     uint32_t m, uint32_t n, uint32_t k)
{
    double *a = (double *)malloc(sizeof(double) * (uint64_t)m * k);
    double *row = (double *)malloc(sizeof(double) * k);
    for (uint64_t i = 0; i < (uint64_t)m * k; ++i) a[i] = oracle_bf16_to_f64(act[i]);
    for (uint64_t j = 0; j < n; ++j) {
        oracle_q4k_decode(w + j * (k / 256u) * 144u, row, 1u, k);
        for (uint64_t i = 0; i < m; ++i) {
            double s = 0.0;
            for (uint64_t kk = 0; kk < k; ++kk) s += a[i * k + kk] * row[kk];
            R[i * n + j] = s;
        }
    }
    free(row);
    free(a);
}

/* Q4_K weight quantization: bf16 [n][k] -> block_q4_K [n][k/256], k a
 * multiple of 256, super-block s of row r at byte (r * k/256 + s) * 144.
 * [page layers/ops/q4k_mmq.rs, fn quantize_weight_q4k: bf16 weights
 *  [nrows, n_per_row] become block_q4_K, one 256-value block per thread; the
 *  module notes that each weight is converted once and cached.]
 * The page names the conversion but prints no rule.  Reading adopted: an
 * affine min/max fit per 32-value sub-block j, whose step and offset are then
 * stored as 6-bit multiples of two fp16 super-block scales.  All arithmetic
 * is binary32 with IEEE division and C roundf (ties away from zero):
 *   lo_j = min(+0, min x)          (the format's offset -dmin*m_j is <= 0)
 *   hi_j = max(lo_j, max x)
 *   S_j  = (hi_j - lo_j) / 15      (step that spans the sub-block)
 *   M_j  = 0 - lo_j                (offset, >= +0)
 *   d    = fp16_rne(max_j S_j / 63), dmin = fp16_rne(max_j M_j / 63)
 *   sc_j = d    > 0 ? min(63, roundf(S_j / d))    : 0
 *   m_j  = dmin > 0 ? min(63, roundf(M_j / dmin)) : 0
 *   q    = clamp(roundf((x + dmin * m_j) / (d * sc_j)), 0, 15),  q = 0 when
 *          d * sc_j == 0.
 * The two products are exact in binary32 (11-bit times 6-bit significands).
 * The maxima start at +0, so no step or scale is a negative zero.  Bytes are
 * then packed in the layout q4k_scale_min and q4k_code read.
 * Returns the number of super-blocks outside the supported range: a value
 * that is not finite, or d or dmin that overflows binary16. */
int64_t oracle_quantize_weight_q4k(const uint16_t *wb, uint8_t *out, uint32_t n, uint32_t k)
{
    uint64_t nsb = k / 256u;
    int64_t flagged = 0;
    for (uint64_t r = 0; r < n; ++r)
        for (uint64_t s = 0; s < nsb; ++s) {
            const uint16_t *src = wb + r * k + s * 256u;
            uint8_t *blk = out + (r * nsb + s) * 144u;
            float x[256], S[8], M[8];
            int bad = 0;
            for (int e = 0; e < 256; ++e) {
                x[e] = (float)oracle_bf16_to_f64(src[e]);
                if (!isfinite(x[e])) bad = 1;
            }
            float maxS = 0.0f, maxM = 0.0f;
            for (int j = 0; j < 8; ++j) {
                float lo = 0.0f;
                for (int i = 0; i < 32; ++i)
                    if (x[32 * j + i] < lo) lo = x[32 * j + i];
                float hi = lo;
                for (int i = 0; i < 32; ++i)
                    if (x[32 * j + i] > hi) hi = x[32 * j + i];
                S[j] = (hi - lo) / 15.0f;
                M[j] = 0.0f - lo;
                if (S[j] > maxS) maxS = S[j];
                if (M[j] > maxM) maxM = M[j];
            }
            uint16_t dh = oracle_f32_to_f16(maxS / 63.0f);
            uint16_t mh = oracle_f32_to_f16(maxM / 63.0f);
            float d = oracle_f16_to_f32(dh), dmin = oracle_f16_to_f32(mh);
            if (!isfinite(d) || !isfinite(dmin)) bad = 1;
            flagged += bad;
            uint32_t sc[8], mn[8];
            for (int j = 0; j < 8; ++j) {
                sc[j] = 0u;
                mn[j] = 0u;
                /* a NaN quotient (only for a block outside the supported
                 * range, whose bytes are unspecified) gives 0 rather than an
                 * undefined float-to-unsigned conversion */
                if (d > 0.0f) {
                    float t = roundf(S[j] / d);
                    sc[j] = !(t > 0.0f) ? 0u : (t > 63.0f ? 63u : (uint32_t)t);
                }
                if (dmin > 0.0f) {
                    float t = roundf(M[j] / dmin);
                    mn[j] = !(t > 0.0f) ? 0u : (t > 63.0f ? 63u : (uint32_t)t);
                }
            }
            /* header: fp16 d, fp16 dmin, then the twelve scale/min bytes */
            blk[0] = (uint8_t)(dh & 0xFFu);
            blk[1] = (uint8_t)(dh >> 8);
            blk[2] = (uint8_t)(mh & 0xFFu);
            blk[3] = (uint8_t)(mh >> 8);
            uint8_t *Sb = blk + 4;
            for (int j = 0; j < 4; ++j) {
                Sb[j] = (uint8_t)((sc[j] & 63u) | ((sc[j + 4] >> 4) << 6));
                Sb[j + 4] = (uint8_t)((mn[j] & 63u) | ((mn[j + 4] >> 4) << 6));
                Sb[j + 8] = (uint8_t)((sc[j + 4] & 15u) | ((mn[j + 4] & 15u) << 4));
            }
            /* codes: chunk t of 64 values, byte 16 + 32t + i holds value
             * 64t + i in the low nibble and 64t + 32 + i in the high nibble */
            memset(blk + 16, 0, 128);
            for (int e = 0; e < 256; ++e) {
                int j = e / 32;
                float step = d * (float)sc[j];
                float off = dmin * (float)mn[j];
                uint32_t q = 0u;
                if (step > 0.0f) {
                    float t = roundf((x[e] + off) / step);
                    q = !(t > 0.0f) ? 0u : (t > 15.0f ? 15u : (uint32_t)t);
                }
                int t64 = e / 64, within = e % 64;
                uint8_t *b = blk + 16 + 32 * t64 + (within % 32);
                *b = (uint8_t)(*b | (within < 32 ? q : (q << 4)));
            }
        }
    return flagged;
}

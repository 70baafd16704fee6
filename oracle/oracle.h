/*
 * CPU oracle for the packed low-bit weight-quantized matmul -- declarations.
 * TEST INFRASTRUCTURE ONLY: see oracle.c.  This header is the oracle's own;
 * the HIP library neither includes it nor shares any of its definitions.
 */
#ifndef BQMM_ORACLE_H
#define BQMM_ORACLE_H
#include <stdint.h>

float oracle_f16_to_f32(uint16_t h);
uint16_t oracle_f32_to_f16(float x);
double oracle_bf16_to_f64(uint16_t b);
uint16_t oracle_f64_to_bf16(double x);

uint64_t oracle_q8_1_kpad(uint32_t k);
uint64_t oracle_q8_1_bytes(uint32_t m, uint32_t k);
int64_t oracle_quantize_act_q8_1(const uint16_t *act, uint8_t *out, uint32_t m, uint32_t k);
void oracle_dequant_q8_1(const uint8_t *q8, double *out, uint32_t m, uint32_t k);

uint64_t oracle_q2_0_bytes(uint32_t n, uint32_t k, uint32_t group);
void oracle_q2_0_decode(const uint8_t *w, double *out, uint32_t n, uint32_t k, uint32_t group);
void oracle_dequant_q2_0_to_bf16(const uint8_t *w, uint16_t *out, uint32_t n, uint32_t k, uint32_t group);
void oracle_q2_0_blockdots(const uint8_t *q8, const uint8_t *w, int32_t *D, uint32_t m, uint32_t n, uint32_t k);
void oracle_q2_0_mmq(const uint8_t *q8, const uint8_t *w, double *R, uint32_t m, uint32_t n, uint32_t k);
void oracle_q2_0_gemv(const uint16_t *act, const uint8_t *w, double *R, uint32_t m, uint32_t n, uint32_t k);
void oracle_dense_gemm_bf16(const uint16_t *a, const uint16_t *w, double *R, uint32_t m, uint32_t n, uint32_t k);
void oracle_silu_mul_bf16(const uint16_t *g, const uint16_t *u, uint16_t *out, uint64_t count);
void oracle_round_bf16(const double *in, uint16_t *out, uint64_t count);

uint64_t oracle_q4k_bytes(uint32_t n, uint32_t k);
void oracle_q4k_decode(const uint8_t *w, double *out, uint32_t n, uint32_t k);
void oracle_q4k_blockdots(const uint8_t *q8, const uint8_t *w, int32_t *D, uint32_t m, uint32_t n, uint32_t k);
void oracle_q4k_mmq(const uint8_t *q8, const uint8_t *w, double *R, uint32_t m, uint32_t n, uint32_t k);
void oracle_q4k_gemv(const uint16_t *act, const uint8_t *w, double *R, uint32_t m, uint32_t n, uint32_t k);
int64_t oracle_quantize_weight_q4k(const uint16_t *wb, uint8_t *out, uint32_t n, uint32_t k);

#endif

// Internal declarations shared by the kernel sources and the C ABI layer.
// gfx950 (CDNA4) only: wave64, int8/bf16 matrix cores, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <tuple>
#include <utility>
#include <vector>

namespace bqmm {

// ---- device helpers ------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// binary32 -> bfloat16 bits, round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// binary32 -> binary16 bits, round to nearest even (v_cvt_f16_f32).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// silu(g) * u = g / (1 + exp(-g)) * u in binary32, with the hardware base-2
// exponential and reciprocal (each within about one ulp, so the product is
// within one bf16 step of the exact value once rounded to bf16; an accurate
// expf and an IEEE division cost about 20 more VALU instructions per value).
// The silu_mul kernel, the fused silu_mul -> q8_1 quantizer and the fused
// gate/up GEMV epilogue share it, so all of them round the same value.
__device__ __forceinline__ float silu_mul_f32(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// ---- host helpers ---------------------------------------------------------

// Raise a kernel's dynamic-LDS limit (beyond the 64 KB default) on the current
// device.  The attribute is per device, so it is set once per (kernel, device)
// and remembered; the lookup takes a lock, which costs far less than a launch.
inline hipError_t ensure_dynamic_lds(const void *kernel, int bytes) {
  static std::mutex mu;
  static std::vector<std::tuple<const void *, int, int>> done;  // kernel, device, bytes
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto &t : done)
    if (std::get<0>(t) == kernel && std::get<1>(t) == dev && std::get<2>(t) >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.emplace_back(kernel, dev, bytes);
  return e;
}

// Compute units of the current device, queried once per device.
inline hipError_t device_cu_count(int *cus) {
  static std::mutex mu;
  static std::vector<std::pair<int, int>> known;  // device, compute units
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto &p : known)
    if (p.first == dev) {
      *cus = p.second;
      return hipSuccess;
    }
  int v = 0;
  e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  known.emplace_back(dev, v);
  *cus = v;
  return hipSuccess;
}

// Batch size from which the batched Q2_0 GEMV (single and fused gate/up) runs
// on matrix cores rather than on the vector ALU; both sources dispatch on it.
#ifndef BQMM_GEMV_MIN_M_MFMA
#define BQMM_GEMV_MIN_M_MFMA 3
#endif

// ---- launchers (one per kernel source) ------------------------------------
// Arguments are validated by the C ABI layer before these are called.

hipError_t launch_quantize_act_q8_1(const void *act, void *out, uint32_t m, uint32_t k,
                                    hipStream_t s);
hipError_t launch_silu_mul_quantize_q8_1(const void *gate, const void *up, void *out, uint32_t m,
                                         uint32_t k, hipStream_t s);
hipError_t launch_dequant_q2_0(const void *w, void *out, uint32_t n, uint32_t k, uint32_t group,
                               hipStream_t s);
hipError_t launch_silu_mul(const void *gate, const void *up, void *out, uint64_t count,
                           hipStream_t s);
hipError_t launch_q2_0_gemv(const void *act, const void *w, void *out, uint32_t m, uint32_t n,
                            uint32_t k, hipStream_t s);
hipError_t launch_q2_0_gemv_gate_up_silu(const void *act, const void *w_gate, const void *w_up,
                                         void *out, uint32_t m, uint32_t n, uint32_t k,
                                         hipStream_t s);
hipError_t launch_q4k_gemv(const void *act, const void *w, void *out, uint32_t n, uint32_t k,
                           hipStream_t s);
hipError_t launch_quantize_weight_q4k(const void *w_bf16, void *out, uint32_t n, uint32_t k,
                                      hipStream_t s);
// True when the matrix-core GEMV's staged weight scales fit 64 KB of LDS for
// this shape (nw = 1 single weight, 2 fused gate/up); the dispatcher falls
// back to the vector kernel otherwise.
bool q2_0_gemv_mfma_fits(uint32_t n, uint32_t k, int nw);
hipError_t launch_q2_0_gemv_mfma(const void *act, const void *w, void *out, uint32_t m, uint32_t n,
                                 uint32_t k, hipStream_t s);
hipError_t launch_q2_0_gemv_mfma_gate_up(const void *act, const void *w_gate, const void *w_up,
                                         void *out, uint32_t m, uint32_t n, uint32_t k,
                                         hipStream_t s);
// ldc: row stride of out in elements (>= n); out row i starts at out + i * ldc
hipError_t launch_q2_0_mmq(const void *act_q8, const void *w, void *out, int32_t *dots,
                           uint32_t m0, uint32_t mt, uint32_t n0, uint32_t nt, uint32_t m,
                           uint32_t n, uint32_t k, uint32_t ldc, hipStream_t s);
hipError_t launch_q4k_mmq(const void *act_q8, const void *w, void *out, int32_t *dots,
                          uint32_t m0, uint32_t mt, uint32_t n0, uint32_t nt, uint32_t m,
                          uint32_t n, uint32_t k, uint32_t ldc, hipStream_t s);
hipError_t launch_dense_gemm_bf16(const void *a, const void *w, void *out, uint32_t m, uint32_t n,
                                  uint32_t k, hipStream_t s);

}  // namespace bqmm

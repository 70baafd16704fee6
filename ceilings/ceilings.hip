// Measured ceilings for the benchmark: what this GPU reaches on the launch,
// streaming-read, int8 matrix-core and vector-ALU paths alone, so that the
// hot path's figures can be read against them as well as against the
// published peaks.  Bench-only: built into its own library, never linked
// into libbqmm.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Nothing: the cost of dispatching a grid and retiring it.
__global__ void empty_kernel() {}

// Reads `bytes` (a multiple of 16) once with 16-byte loads: workgroup b
// takes the b-th of gridDim.x equal contiguous ranges, and each lane issues
// all of its (at most kLoads) loads before using any, so every load of a
// launch is in flight at once (lanes past the range's end load its last
// chunk again).  The loaded words are folded together and stored only if the
// fold hits a value that the inputs here never produce, so the loads cannot
// be dropped and (in practice) nothing is written.
constexpr int kLoads = 4;
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *__restrict__ src, uint64_t chunks,
                                                          uint32_t *__restrict__ sink) {
  const uint64_t per = (chunks + gridDim.x - 1) / gridDim.x;
  const uint64_t begin = (uint64_t)blockIdx.x * per;
  const uint64_t end = begin + per < chunks ? begin + per : chunks;
  if (begin >= end) return;
  uint4 v[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const uint64_t i = begin + threadIdx.x + (uint64_t)j * blockDim.x;
    v[j] = src[i < end ? i : end - 1];
  }
  uint32_t x = 0;
#pragma unroll
  for (int j = 0; j < kLoads; ++j) x ^= v[j].x ^ (v[j].y * 3u) ^ (v[j].z * 5u) ^ (v[j].w * 7u);
  if (x == 0x9E3779B9u) sink[blockIdx.x] = x;
}

// The same read, then every workgroup writes its share of `outs` 2-byte
// values (the decode GEMV's output: one bf16 per weight row), each a fold of
// the lane's loaded words: the GEMV's whole memory traffic with its grid,
// and no arithmetic.
__global__ __launch_bounds__(256) void stream_read_write_kernel(const uint4 *__restrict__ src, uint64_t chunks,
                                                                uint16_t *__restrict__ dst, uint32_t outs) {
  const uint64_t per = (chunks + gridDim.x - 1) / gridDim.x;
  const uint64_t begin = (uint64_t)blockIdx.x * per;
  const uint64_t end = begin + per < chunks ? begin + per : chunks;
  uint32_t x = 0;
  if (begin < end) {
    uint4 v[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const uint64_t i = begin + threadIdx.x + (uint64_t)j * blockDim.x;
      v[j] = src[i < end ? i : end - 1];
    }
#pragma unroll
    for (int j = 0; j < kLoads; ++j) x ^= v[j].x ^ (v[j].y * 3u) ^ (v[j].z * 5u) ^ (v[j].w * 7u);
  }
  const uint32_t per_out = (outs + gridDim.x - 1) / gridDim.x;
  const uint32_t o = blockIdx.x * per_out + threadIdx.x;
  if (threadIdx.x < per_out && o < outs) dst[o] = (uint16_t)(x & 0x7FFFu);
}

// Back-to-back v_mfma_i32_32x32x32_i8 with four independent accumulators per
// wave (no dependent chain, no memory traffic in the loop): the int8 matrix
// core's issue rate.
__global__ __launch_bounds__(256) void mfma_i8_kernel(uint32_t iters, int seed, int *__restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const v4i a = {seed + lane, seed ^ lane, seed - lane, seed * 3 + lane};
  const v4i b = {lane, seed, lane * 5, seed - 7};
  v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (uint32_t i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) s ^= c0[r] ^ c1[r] ^ c2[r] ^ c3[r];
  if (s == 0x7FEDCBA9) sink[blockIdx.x] = s;
}

// The same for v_mfma_f32_32x32x16_f16, the instruction the Q4_K MMQ runs on:
// the fp16 matrix core's issue rate.
__global__ __launch_bounds__(256) void mfma_f16_kernel(uint32_t iters, int seed, int *__restrict__ sink) {
  const int lane = threadIdx.x & 63;
  v8h a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (_Float16)(float)((seed + lane + j) & 7);
    b[j] = (_Float16)(float)((lane * 3 + j) & 7);
  }
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (uint32_t i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  if (s == -1.0f) sink[blockIdx.x] = (int)s;
}

// Independent chains of the integer multiply-add the Q2_0 MMQ folds with
// (v_mad_i32_i24): eight chains per lane, so each instruction's result is
// not awaited by the next; the vector ALU's issue rate.
__global__ __launch_bounds__(256) void valu_mad_kernel(uint32_t iters, int seed, int *__restrict__ sink) {
  const int t = (int)threadIdx.x;
  int a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = seed + t * (j + 1);
  const int m0 = (seed & 0x7FF) + 3, m1 = ((seed >> 3) & 0x7FF) + 5;
  for (uint32_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = ((a[j] << 8) >> 8) * (((j & 1) ? m0 : m1)) + a[j];
  }
  int s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) s ^= a[j];
  if (s == 0x7FEDCBA9) sink[blockIdx.x] = s;
}

// MFMAs and vector-ALU work in one instruction stream: per iteration four
// independent MFMAs (int8 32x32x32, or fp16 32x32x16 when kF16) and kV
// 24-bit multiply-adds in eight independent chains, so neither unit waits on
// the other's results: what the chip sustains at a given mix of VALU
// instructions per MFMA (the MMQ kernels' fold and staging work per MFMA).
template <bool kF16, int kV>
__global__ __launch_bounds__(256) void mix_kernel(uint32_t iters, int seed, int *__restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const v4i a = {seed + lane, seed ^ lane, seed - lane, seed * 3 + lane};
  const v4i b = {lane, seed, lane * 5, seed - 7};
  v8h ah, bh;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ah[j] = (_Float16)(float)((seed + lane + j) & 7);
    bh[j] = (_Float16)(float)((lane * 3 + j) & 7);
  }
  v16i c[4] = {};
  v16f f[4] = {};
  int x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = seed + lane * (j + 1);
  const int m0 = (seed & 0x7FF) + 3;
  for (uint32_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (kF16)
        f[q] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, f[q], 0, 0, 0);
      else
        c[q] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[q], 0, 0, 0);
#pragma unroll
      for (int v = 0; v < kV / 4; ++v) x[v & 7] = ((x[v & 7] << 8) >> 8) * m0 + x[v & 7];
    }
  }
  int s = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) s ^= c[q][r] ^ (int)f[q][r];
#pragma unroll
  for (int j = 0; j < 8; ++j) s ^= x[j];
  if (s == 0x7FEDCBA9) sink[blockIdx.x] = s;
}

// LDS bandwidth: each lane reads (or writes) 16 consecutive bytes per access,
// a wave 1 KiB without bank conflicts, 16 accesses per iteration over a
// 64 KiB buffer (two workgroups per CU).
template <bool kWrite>
__global__ __launch_bounds__(256) void lds_kernel(uint32_t iters, int *__restrict__ sink) {
  __shared__ uint4 buf[4096];
  const uint32_t t = threadIdx.x;
  for (uint32_t i = t; i < 4096u; i += 256u) buf[i] = make_uint4(i, i * 3u, i * 7u, i * 11u);
  __syncthreads();
  uint32_t acc = 0, acc2 = 0;
  for (uint32_t it = 0; it < iters; ++it) {
    const uint32_t sh = (it & 7u) * 256u;
    const uint4 d = make_uint4(it, t, acc, 7u);
#pragma unroll
    for (uint32_t i = 0; i < 16u; ++i) {
      const uint32_t idx = (t + 256u * i + sh) & 4095u;
      if (kWrite) {
        buf[idx] = d;
      } else {
        // two three-input adds per access keep the vector ALU off the path
        const uint4 v = buf[idx];
        acc = acc + v.x + v.y;
        acc2 = acc2 + v.z + v.w;
      }
    }
  }
  __syncthreads();
  acc ^= acc2 ^ buf[t].x;
  if (acc == 0x7FEDCBA9u) sink[blockIdx.x] = (int)acc;
}

}  // namespace

extern "C" {

// Each launches one kernel on `stream` and returns the HIP status.
int ceil_empty(uint32_t blocks, uint32_t threads, void *stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(blocks), dim3(threads), 0, static_cast<hipStream_t>(stream));
  return (int)hipGetLastError();
}

// bytes % 16 == 0 and bytes <= blocks * 256 * kLoads * 16 (every chunk read);
// sink holds `blocks` uint32.
int ceil_stream_read(const void *src, uint64_t bytes, void *sink, uint32_t blocks, void *stream) {
  if (bytes % 16u != 0 || bytes > (uint64_t)blocks * 256u * kLoads * 16u) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4 *>(src), bytes / 16u, static_cast<uint32_t *>(sink));
  return (int)hipGetLastError();
}

// As ceil_stream_read, then `outs` 2-byte values written to dst (outs <= blocks * 256).
int ceil_stream_read_write(const void *src, uint64_t bytes, void *dst, uint32_t outs, uint32_t blocks,
                           void *stream) {
  if (bytes % 16u != 0 || bytes > (uint64_t)blocks * 256u * kLoads * 16u || outs > blocks * 256u)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_write_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4 *>(src), bytes / 16u, static_cast<uint16_t *>(dst), outs);
  return (int)hipGetLastError();
}

// Work per launch: blocks * 4 waves * iters * 4 MFMAs * 2*32*32*32 int8 ops.
int ceil_mfma_i8(uint32_t blocks, uint32_t iters, void *sink, void *stream) {
  hipLaunchKernelGGL(mfma_i8_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters, 12345,
                     static_cast<int *>(sink));
  return (int)hipGetLastError();
}

// Work per launch: blocks * 4 waves * iters * 4 MFMAs * 2*32*32*16 fp16 flops.
int ceil_mfma_f16(uint32_t blocks, uint32_t iters, void *sink, void *stream) {
  hipLaunchKernelGGL(mfma_f16_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters, 12345,
                     static_cast<int *>(sink));
  return (int)hipGetLastError();
}

// Work per launch: blocks * 4 waves * iters * 4 MFMAs (int8 32x32x32, or
// fp16 32x32x16 when f16 != 0) plus valu_per_4 wave-wide multiply-adds per 4
// MFMAs; valu_per_4 is one of 96, 132 (int8) or 56 (fp16).
int ceil_mix(uint32_t blocks, uint32_t iters, int f16, uint32_t valu_per_4, void *sink, void *stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  int *k = static_cast<int *>(sink);
  if (!f16 && valu_per_4 == 96u)
    hipLaunchKernelGGL((mix_kernel<false, 96>), dim3(blocks), dim3(256), 0, s, iters, 12345, k);
  else if (!f16 && valu_per_4 == 132u)
    hipLaunchKernelGGL((mix_kernel<false, 132>), dim3(blocks), dim3(256), 0, s, iters, 12345, k);
  else if (f16 && valu_per_4 == 56u)
    hipLaunchKernelGGL((mix_kernel<true, 56>), dim3(blocks), dim3(256), 0, s, iters, 12345, k);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

// Bytes per launch: blocks * 256 lanes * iters * 16 accesses * 16 bytes.
int ceil_lds(uint32_t blocks, uint32_t iters, int write, void *sink, void *stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (write)
    hipLaunchKernelGGL(lds_kernel<true>, dim3(blocks), dim3(256), 0, s, iters, static_cast<int *>(sink));
  else
    hipLaunchKernelGGL(lds_kernel<false>, dim3(blocks), dim3(256), 0, s, iters, static_cast<int *>(sink));
  return (int)hipGetLastError();
}

// Work per launch: blocks * 4 waves * iters * 8 wave-wide multiply-adds.
int ceil_valu_mad(uint32_t blocks, uint32_t iters, void *sink, void *stream) {
  hipLaunchKernelGGL(valu_mad_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters, 777,
                     static_cast<int *>(sink));
  return (int)hipGetLastError();
}

}  // extern "C"

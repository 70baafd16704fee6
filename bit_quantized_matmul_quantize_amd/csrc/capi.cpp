// The C ABI: argument checks, then one launch (or two, for the dispatcher) on
// the caller's stream.  Every check runs before any HIP call.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/bqmm.h"
#include "bqmm_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(BQ_EHIP, "%s: %s", what, hipGetErrorString(e));
  g_last_error[0] = '\0';
  return BQ_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0u; }

// True when the byte ranges [a, a + na) and [b, b + nb) share a byte.
bool overlap(const void *a, uint64_t na, const void *b, uint64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

uint64_t q8_bytes(uint32_t m, uint32_t k) {
  const uint64_t kpad = ((uint64_t)k + 255u) / 256u * 256u;
  return (uint64_t)m * kpad + (uint64_t)m * (kpad / 32u) * 4u;
}

uint64_t q2_bytes(uint32_t n, uint32_t k) { return (uint64_t)n * k / 4u + 2u * (uint64_t)n * (k / 128u); }

uint64_t q4k_bytes(uint32_t n, uint32_t k) { return (uint64_t)n * (k / 256u) * 144u; }

uint64_t bf16_bytes(uint64_t rows, uint64_t cols) { return 2u * rows * cols; }

// bytes spanned by rows of n bf16 values at a row stride of ldc values
uint64_t strided_bytes(uint32_t m, uint32_t n, uint32_t ldc) { return 2u * ((uint64_t)(m - 1u) * ldc + n); }

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

constexpr uint32_t kMaxGridY = 65535u;
// Bounds that keep every size and index computation inside its type: k values
// per row (padded to 256 in 32 bits), and output rows n.
constexpr uint32_t kMaxK = 1u << 30;
constexpr uint32_t kMaxRows = 1u << 31;

#define REQUIRE(cond, status, ...) \
  do {                             \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

// Output buffers must not overlap inputs (the kernels read inputs while other
// workgroups write the output).
#define REQUIRE_DISJOINT(name, out, nout, in, nin, what)                                      \
  REQUIRE(!overlap(out, nout, in, nin), BQ_EINVAL, "%s: the output overlaps %s", name, what)

}  // namespace

extern "C" {

const char *bq_last_error(void) { return g_last_error; }

const char *bq_status_string(int status) {
  switch (status) {
    case BQ_OK: return "ok";
    case BQ_EINVAL: return "invalid argument";
    case BQ_EUNSUPPORTED: return "unsupported configuration";
    case BQ_EALIGN: return "pointer not 16-byte aligned";
    case BQ_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

uint64_t q8_1_act_bytes(uint32_t m, uint32_t k) {
  const uint64_t kpad = ((uint64_t)k + 255u) / 256u * 256u;
  return (uint64_t)m * kpad + (uint64_t)m * (kpad / 32u) * 4u;
}

uint64_t q2_0_weight_bytes(uint32_t n, uint32_t k, uint32_t group) {
  if (group == 0 || group % 32u != 0 || k % group != 0) return 0;
  return (uint64_t)n * k / 4u + 2u * (uint64_t)n * (k / group);
}

uint64_t q4k_weight_bytes(uint32_t n, uint32_t k) {
  if (k % 256u != 0) return 0;
  return (uint64_t)n * (k / 256u) * 144u;
}

int quantize_act_q8_1(const void *act_bf16, void *out_q8, uint32_t m, uint32_t k, void *stream) {
  REQUIRE(act_bf16 && out_q8, BQ_EINVAL, "quantize_act_q8_1: null pointer");
  REQUIRE(m >= 1 && k >= 1, BQ_EINVAL, "quantize_act_q8_1: m=%u k=%u must be >= 1", m, k);
  REQUIRE(k <= kMaxK, BQ_EINVAL, "quantize_act_q8_1: k=%u too large", k);
  REQUIRE(aligned16(act_bf16) && aligned16(out_q8), BQ_EALIGN, "quantize_act_q8_1: buffers must be 16-byte aligned");
  const uint64_t kpad = ((uint64_t)k + 255u) / 256u * 256u;
  const uint64_t blocks = (uint64_t)m * ((kpad + 2047u) / 2048u);
  REQUIRE(blocks < (1ull << 31), BQ_EINVAL, "quantize_act_q8_1: m*k too large");
  REQUIRE_DISJOINT("quantize_act_q8_1", out_q8, q8_bytes(m, k), act_bf16, bf16_bytes(m, k), "the input");
  return hip_status(bqmm::launch_quantize_act_q8_1(act_bf16, out_q8, m, k, as_stream(stream)),
                    "quantize_act_q8_1");
}

int silu_mul_quantize_q8_1(const void *gate_bf16, const void *up_bf16, void *out_q8, uint32_t m,
                           uint32_t k, void *stream) {
  REQUIRE(gate_bf16 && up_bf16 && out_q8, BQ_EINVAL, "silu_mul_quantize_q8_1: null pointer");
  REQUIRE(m >= 1 && k >= 1, BQ_EINVAL, "silu_mul_quantize_q8_1: m=%u k=%u must be >= 1", m, k);
  REQUIRE(k <= kMaxK, BQ_EINVAL, "silu_mul_quantize_q8_1: k=%u too large", k);
  REQUIRE(aligned16(gate_bf16) && aligned16(up_bf16) && aligned16(out_q8), BQ_EALIGN,
          "silu_mul_quantize_q8_1: buffers must be 16-byte aligned");
  const uint64_t kpad = ((uint64_t)k + 255u) / 256u * 256u;
  const uint64_t blocks = (uint64_t)m * ((kpad + 2047u) / 2048u);
  REQUIRE(blocks < (1ull << 31), BQ_EINVAL, "silu_mul_quantize_q8_1: m*k too large");
  REQUIRE_DISJOINT("silu_mul_quantize_q8_1", out_q8, q8_bytes(m, k), gate_bf16, bf16_bytes(m, k), "gate");
  REQUIRE_DISJOINT("silu_mul_quantize_q8_1", out_q8, q8_bytes(m, k), up_bf16, bf16_bytes(m, k), "up");
  return hip_status(bqmm::launch_silu_mul_quantize_q8_1(gate_bf16, up_bf16, out_q8, m, k, as_stream(stream)),
                    "silu_mul_quantize_q8_1");
}

// out_bytes: the span the call writes (0 = the plain [m][n] bf16 output;
// ~0 = no range check here, the caller does it after its own checks)
static int check_mmq(const char *name, const void *act_q8, const void *w, const void *out,
                     uint32_t m, uint32_t n, uint32_t k, uint32_t kmult, uint64_t out_bytes = 0) {
  REQUIRE(act_q8 && w && out, BQ_EINVAL, "%s: null pointer", name);
  REQUIRE(m >= 1 && n >= 1 && k >= 1, BQ_EINVAL, "%s: m=%u n=%u k=%u must be >= 1", name, m, n, k);
  REQUIRE(k % kmult == 0, BQ_EINVAL, "%s: k=%u must be a multiple of %u", name, k, kmult);
  REQUIRE(aligned16(act_q8) && aligned16(w) && aligned16(out), BQ_EALIGN, "%s: buffers must be 16-byte aligned", name);
  REQUIRE(k <= kMaxK && n <= kMaxRows, BQ_EINVAL, "%s: n=%u k=%u too large", name, n, k);
  REQUIRE(((uint64_t)m + 127u) / 128u <= kMaxGridY, BQ_EINVAL, "%s: m=%u too large", name, m);
  if (out_bytes == ~0ull) return BQ_OK;  // the caller checks the ranges itself
  const uint64_t nout = out_bytes ? out_bytes : bf16_bytes(m, n);
  REQUIRE_DISJOINT(name, out, nout, act_q8, q8_bytes(m, k), "the q8_1 activations");
  REQUIRE_DISJOINT(name, out, nout, w, kmult == 256u ? q4k_bytes(n, k) : q2_bytes(n, k), "the weight");
  return BQ_OK;
}

int q2_0_mmq_gemm(const void *act_q8, const void *w_q2, void *out_bf16, uint32_t m, uint32_t n,
                  uint32_t k, void *stream) {
  const int st = check_mmq("q2_0_mmq_gemm", act_q8, w_q2, out_bf16, m, n, k, 128u);
  if (st != BQ_OK) return st;
  return hip_status(bqmm::launch_q2_0_mmq(act_q8, w_q2, out_bf16, nullptr, 0, 0, 0, 0, m, n, k, n,
                                          as_stream(stream)),
                    "q2_0_mmq_gemm");
}

int q2_0_mmq_gemm_ldc(const void *act_q8, const void *w_q2, void *out_bf16, uint32_t m, uint32_t n,
                      uint32_t k, uint32_t ldc, void *stream) {
  REQUIRE(ldc >= n, BQ_EINVAL, "q2_0_mmq_gemm_ldc: ldc=%u must be >= n=%u", ldc, n);
  const int st = check_mmq("q2_0_mmq_gemm_ldc", act_q8, w_q2, out_bf16, m, n, k, 128u,
                           m >= 1 && n >= 1 ? strided_bytes(m, n, ldc) : 0);
  if (st != BQ_OK) return st;
  return hip_status(bqmm::launch_q2_0_mmq(act_q8, w_q2, out_bf16, nullptr, 0, 0, 0, 0, m, n, k, ldc,
                                          as_stream(stream)),
                    "q2_0_mmq_gemm_ldc");
}

int q4k_mmq_gemm(const void *act_q8, const void *w_q4k, void *out_bf16, uint32_t m, uint32_t n,
                 uint32_t k, void *stream) {
  const int st = check_mmq("q4k_mmq_gemm", act_q8, w_q4k, out_bf16, m, n, k, 256u);
  if (st != BQ_OK) return st;
  return hip_status(bqmm::launch_q4k_mmq(act_q8, w_q4k, out_bf16, nullptr, 0, 0, 0, 0, m, n, k, n,
                                         as_stream(stream)),
                    "q4k_mmq_gemm");
}

int q4k_mmq_gemm_ldc(const void *act_q8, const void *w_q4k, void *out_bf16, uint32_t m, uint32_t n,
                     uint32_t k, uint32_t ldc, void *stream) {
  REQUIRE(ldc >= n, BQ_EINVAL, "q4k_mmq_gemm_ldc: ldc=%u must be >= n=%u", ldc, n);
  const int st = check_mmq("q4k_mmq_gemm_ldc", act_q8, w_q4k, out_bf16, m, n, k, 256u,
                           m >= 1 && n >= 1 ? strided_bytes(m, n, ldc) : 0);
  if (st != BQ_OK) return st;
  return hip_status(bqmm::launch_q4k_mmq(act_q8, w_q4k, out_bf16, nullptr, 0, 0, 0, 0, m, n, k, ldc,
                                         as_stream(stream)),
                    "q4k_mmq_gemm_ldc");
}

static int check_blockdots(const char *name, const void *act_q8, const void *w, const int32_t *out,
                           uint32_t m0, uint32_t mt, uint32_t n0, uint32_t nt, uint32_t m, uint32_t n,
                           uint32_t k, uint32_t kmult) {
  int st = check_mmq(name, act_q8, w, out, m, n, k, kmult, ~0ull);
  if (st != BQ_OK) return st;
  REQUIRE(mt >= 1 && nt >= 1, BQ_EINVAL, "%s: empty window", name);
  REQUIRE((uint64_t)m0 + mt <= m && (uint64_t)n0 + nt <= n, BQ_EINVAL,
          "%s: window [%u,+%u) x [%u,+%u) outside [0,%u) x [0,%u)", name, m0, mt, n0, nt, m, n);
  // the window's block dots as int32, then the usual rule: no overlap with the inputs
  return check_mmq(name, act_q8, w, out, m, n, k, kmult, 4u * (uint64_t)mt * nt * (k / 32u));
}

int q2_0_mmq_blockdots(const void *act_q8, const void *w_q2, int32_t *out, uint32_t m0, uint32_t mt,
                       uint32_t n0, uint32_t nt, uint32_t m, uint32_t n, uint32_t k, void *stream) {
  const int st = check_blockdots("q2_0_mmq_blockdots", act_q8, w_q2, out, m0, mt, n0, nt, m, n, k, 128u);
  if (st != BQ_OK) return st;
  return hip_status(bqmm::launch_q2_0_mmq(act_q8, w_q2, nullptr, out, m0, mt, n0, nt, m, n, k, n,
                                          as_stream(stream)),
                    "q2_0_mmq_blockdots");
}

int q4k_mmq_blockdots(const void *act_q8, const void *w_q4k, int32_t *out, uint32_t m0, uint32_t mt,
                      uint32_t n0, uint32_t nt, uint32_t m, uint32_t n, uint32_t k, void *stream) {
  const int st = check_blockdots("q4k_mmq_blockdots", act_q8, w_q4k, out, m0, mt, n0, nt, m, n, k, 256u);
  if (st != BQ_OK) return st;
  return hip_status(bqmm::launch_q4k_mmq(act_q8, w_q4k, nullptr, out, m0, mt, n0, nt, m, n, k, n,
                                         as_stream(stream)),
                    "q4k_mmq_blockdots");
}

static int check_gemv(const char *name, const void *act, const void *w, const void *out, uint32_t m,
                      uint32_t n, uint32_t k) {
  REQUIRE(act && w && out, BQ_EINVAL, "%s: null pointer", name);
  REQUIRE(n >= 1 && k >= 1, BQ_EINVAL, "%s: n=%u k=%u must be >= 1", name, n, k);
  REQUIRE(k % 128u == 0, BQ_EINVAL, "%s: k=%u must be a multiple of the group size 128", name, k);
  REQUIRE(k <= kMaxK && n <= kMaxRows, BQ_EINVAL, "%s: n=%u k=%u too large", name, n, k);
  REQUIRE(m >= 1, BQ_EINVAL, "%s: m must be >= 1", name);
  REQUIRE(m <= 8, BQ_EUNSUPPORTED, "%s: m=%u > 8 (use the MMQ path)", name, m);
  REQUIRE(aligned16(act) && aligned16(w) && aligned16(out), BQ_EALIGN, "%s: buffers must be 16-byte aligned", name);
  REQUIRE_DISJOINT(name, out, bf16_bytes(m, n), act, bf16_bytes(m, k), "the activations");
  REQUIRE_DISJOINT(name, out, bf16_bytes(m, n), w, q2_bytes(n, k), "the weight");
  return BQ_OK;
}

int q2_0_gemv_vec(const void *act_bf16, const void *w_q2, void *out_bf16, uint32_t n, uint32_t k,
                  void *stream) {
  const int st = check_gemv("q2_0_gemv_vec", act_bf16, w_q2, out_bf16, 1, n, k);
  if (st != BQ_OK) return st;
  return hip_status(bqmm::launch_q2_0_gemv(act_bf16, w_q2, out_bf16, 1, n, k, as_stream(stream)),
                    "q2_0_gemv_vec");
}

int q2_0_gemv_vec_batchm(const void *act_bf16, const void *w_q2, void *out_bf16, uint32_t m,
                         uint32_t n, uint32_t k, void *stream) {
  const int st = check_gemv("q2_0_gemv_vec_batchm", act_bf16, w_q2, out_bf16, m, n, k);
  if (st != BQ_OK) return st;
  return hip_status(bqmm::launch_q2_0_gemv(act_bf16, w_q2, out_bf16, m, n, k, as_stream(stream)),
                    "q2_0_gemv_vec_batchm");
}

int q2_0_gemv_gate_up_silu(const void *act_bf16, const void *w_gate_q2, const void *w_up_q2,
                           void *out_bf16, uint32_t m, uint32_t n, uint32_t k, void *stream) {
  int st = check_gemv("q2_0_gemv_gate_up_silu", act_bf16, w_gate_q2, out_bf16, m, n, k);
  if (st != BQ_OK) return st;
  REQUIRE(w_up_q2, BQ_EINVAL, "q2_0_gemv_gate_up_silu: null pointer");
  REQUIRE(aligned16(w_up_q2), BQ_EALIGN, "q2_0_gemv_gate_up_silu: buffers must be 16-byte aligned");
  REQUIRE_DISJOINT("q2_0_gemv_gate_up_silu", out_bf16, bf16_bytes(m, n), w_up_q2, q2_bytes(n, k), "the up weight");
  return hip_status(bqmm::launch_q2_0_gemv_gate_up_silu(act_bf16, w_gate_q2, w_up_q2, out_bf16, m, n, k,
                                                        as_stream(stream)),
                    "q2_0_gemv_gate_up_silu");
}

int q4k_gemv_vec(const void *act_bf16, const void *w_q4k, void *out_bf16, uint32_t n, uint32_t k,
                 void *stream) {
  REQUIRE(act_bf16 && w_q4k && out_bf16, BQ_EINVAL, "q4k_gemv_vec: null pointer");
  REQUIRE(n >= 1 && k >= 1, BQ_EINVAL, "q4k_gemv_vec: n=%u k=%u must be >= 1", n, k);
  REQUIRE(k % 256u == 0, BQ_EINVAL, "q4k_gemv_vec: k=%u must be a multiple of 256", k);
  REQUIRE(k <= kMaxK && n <= kMaxRows, BQ_EINVAL, "q4k_gemv_vec: n=%u k=%u too large", n, k);
  REQUIRE(aligned16(act_bf16) && aligned16(w_q4k) && aligned16(out_bf16), BQ_EALIGN,
          "q4k_gemv_vec: buffers must be 16-byte aligned");
  REQUIRE_DISJOINT("q4k_gemv_vec", out_bf16, bf16_bytes(1, n), act_bf16, bf16_bytes(1, k), "the activations");
  REQUIRE_DISJOINT("q4k_gemv_vec", out_bf16, bf16_bytes(1, n), w_q4k, q4k_bytes(n, k), "the weight");
  return hip_status(bqmm::launch_q4k_gemv(act_bf16, w_q4k, out_bf16, n, k, as_stream(stream)), "q4k_gemv_vec");
}

int quantize_weight_q4k(const void *w_bf16, void *out_q4k, uint32_t n, uint32_t k, void *stream) {
  REQUIRE(w_bf16 && out_q4k, BQ_EINVAL, "quantize_weight_q4k: null pointer");
  REQUIRE(n >= 1 && k >= 1, BQ_EINVAL, "quantize_weight_q4k: n=%u k=%u must be >= 1", n, k);
  REQUIRE(k % 256u == 0, BQ_EINVAL, "quantize_weight_q4k: k=%u must be a multiple of 256", k);
  REQUIRE(k <= kMaxK && n <= kMaxRows, BQ_EINVAL, "quantize_weight_q4k: n=%u k=%u too large", n, k);
  // eight lanes per super-block, 256 lanes per workgroup, one grid dimension
  REQUIRE(((uint64_t)n * (k / 256u) * 8u + 255u) / 256u < (1ull << 31), BQ_EINVAL,
          "quantize_weight_q4k: n=%u k=%u too large", n, k);
  REQUIRE(aligned16(w_bf16) && aligned16(out_q4k), BQ_EALIGN,
          "quantize_weight_q4k: buffers must be 16-byte aligned");
  REQUIRE_DISJOINT("quantize_weight_q4k", out_q4k, q4k_bytes(n, k), w_bf16, bf16_bytes(n, k), "the input");
  return hip_status(bqmm::launch_quantize_weight_q4k(w_bf16, out_q4k, n, k, as_stream(stream)),
                    "quantize_weight_q4k");
}

static int check_dequant(const void *w, const void *out, uint32_t n, uint32_t k, uint32_t group) {
  REQUIRE(w && out, BQ_EINVAL, "dequant_q2_0_to_bf16: null pointer");
  REQUIRE(n >= 1 && k >= 1, BQ_EINVAL, "dequant_q2_0_to_bf16: n=%u k=%u must be >= 1", n, k);
  REQUIRE(group >= 32u && group % 32u == 0, BQ_EUNSUPPORTED,
          "dequant_q2_0_to_bf16: group=%u must be a positive multiple of 32", group);
  REQUIRE(k % group == 0, BQ_EINVAL, "dequant_q2_0_to_bf16: k=%u not a multiple of group=%u", k, group);
  REQUIRE(k <= kMaxK && n <= kMaxRows, BQ_EINVAL, "dequant_q2_0_to_bf16: n=%u k=%u too large", n, k);
  REQUIRE(aligned16(w) && aligned16(out), BQ_EALIGN, "dequant_q2_0_to_bf16: buffers must be 16-byte aligned");
  REQUIRE_DISJOINT("dequant_q2_0_to_bf16", out, bf16_bytes(n, k), w,
                   (uint64_t)n * k / 4u + 2u * (uint64_t)n * (k / group), "the weight");
  return BQ_OK;
}

int dequant_q2_0_to_bf16(const void *w_q2, void *out_bf16, uint32_t n, uint32_t k, uint32_t group,
                         void *stream) {
  const int st = check_dequant(w_q2, out_bf16, n, k, group);
  if (st != BQ_OK) return st;
  return hip_status(bqmm::launch_dequant_q2_0(w_q2, out_bf16, n, k, group, as_stream(stream)),
                    "dequant_q2_0_to_bf16");
}

static int check_dense(const void *a, const void *w, const void *out, uint32_t m, uint32_t n, uint32_t k) {
  REQUIRE(a && w && out, BQ_EINVAL, "dense_gemm_bf16: null pointer");
  REQUIRE(m >= 1 && n >= 1 && k >= 1, BQ_EINVAL, "dense_gemm_bf16: m=%u n=%u k=%u must be >= 1", m, n, k);
  REQUIRE(k % 64u == 0, BQ_EINVAL, "dense_gemm_bf16: k=%u must be a multiple of 64", k);
  REQUIRE(aligned16(a) && aligned16(w) && aligned16(out), BQ_EALIGN, "dense_gemm_bf16: buffers must be 16-byte aligned");
  REQUIRE(k <= kMaxK && m <= kMaxRows, BQ_EINVAL, "dense_gemm_bf16: m=%u k=%u too large", m, k);
  REQUIRE(((uint64_t)n + 127u) / 128u <= kMaxGridY, BQ_EINVAL, "dense_gemm_bf16: n=%u too large", n);
  REQUIRE_DISJOINT("dense_gemm_bf16", out, bf16_bytes(m, n), a, bf16_bytes(m, k), "the activations");
  REQUIRE_DISJOINT("dense_gemm_bf16", out, bf16_bytes(m, n), w, bf16_bytes(n, k), "the weight");
  return BQ_OK;
}

int dense_gemm_bf16(const void *a_bf16, const void *w_bf16, void *out_bf16, uint32_t m, uint32_t n,
                    uint32_t k, void *stream) {
  const int st = check_dense(a_bf16, w_bf16, out_bf16, m, n, k);
  if (st != BQ_OK) return st;
  return hip_status(bqmm::launch_dense_gemm_bf16(a_bf16, w_bf16, out_bf16, m, n, k, as_stream(stream)),
                    "dense_gemm_bf16");
}

// Checks of the prefill dispatcher's arguments; the branch's workspace
// (act_q8 for MMQ, scratch_bf16 for the dequant branch) must be given.
static int check_prefill(const char *name, const void *act_bf16, const void *w_q2, const void *out_bf16,
                         const void *scratch_bf16, const void *act_q8, uint32_t m, uint32_t n, uint32_t k,
                         uint32_t group, bool mmq) {
  REQUIRE(act_bf16 && w_q2 && out_bf16, BQ_EINVAL, "%s: null input, weight or output", name);
  if (mmq) {
    REQUIRE(act_q8, BQ_EINVAL, "%s: MMQ branch needs the act_q8 buffer", name);
    REQUIRE(m >= 1 && k >= 1, BQ_EINVAL, "%s: m=%u k=%u must be >= 1", name, m, k);
    REQUIRE(aligned16(act_bf16), BQ_EALIGN, "%s: input must be 16-byte aligned", name);
    const int st = check_mmq(name, act_q8, w_q2, out_bf16, m, n, k, 128u);
    if (st != BQ_OK) return st;
    REQUIRE_DISJOINT(name, act_q8, q8_bytes(m, k), act_bf16, bf16_bytes(m, k), "the input");
    REQUIRE_DISJOINT(name, act_q8, q8_bytes(m, k), w_q2, q2_bytes(n, k), "the weight");
    return BQ_OK;
  }
  REQUIRE(scratch_bf16, BQ_EINVAL, "%s: dequant branch needs the bf16 scratch buffer", name);
  int st = check_dequant(w_q2, scratch_bf16, n, k, group);
  if (st != BQ_OK) return st;
  st = check_dense(act_bf16, scratch_bf16, out_bf16, m, n, k);
  if (st != BQ_OK) return st;
  REQUIRE_DISJOINT(name, scratch_bf16, bf16_bytes(n, k), act_bf16, bf16_bytes(m, k), "the input");
  REQUIRE_DISJOINT(name, out_bf16, bf16_bytes(m, n), w_q2,
                   (uint64_t)n * k / 4u + 2u * (uint64_t)n * (k / group), "the weight");
  return BQ_OK;
}

// The prefill dispatcher's launches, after check_prefill.
static int launch_prefill(const char *name, const void *act_bf16, const void *w_q2, void *out_bf16,
                          void *scratch_bf16, void *act_q8, uint32_t m, uint32_t n, uint32_t k, uint32_t group,
                          bool mmq, hipStream_t s) {
  char what[96];
  if (mmq) {
    std::snprintf(what, sizeof(what), "%s (quantize)", name);
    const int st = hip_status(bqmm::launch_quantize_act_q8_1(act_bf16, act_q8, m, k, s), what);
    if (st != BQ_OK) return st;
    std::snprintf(what, sizeof(what), "%s (mmq)", name);
    return hip_status(bqmm::launch_q2_0_mmq(act_q8, w_q2, out_bf16, nullptr, 0, 0, 0, 0, m, n, k, n, s), what);
  }
  std::snprintf(what, sizeof(what), "%s (dequant)", name);
  const int st = hip_status(bqmm::launch_dequant_q2_0(w_q2, scratch_bf16, n, k, group, s), what);
  if (st != BQ_OK) return st;
  std::snprintf(what, sizeof(what), "%s (dense gemm)", name);
  return hip_status(bqmm::launch_dense_gemm_bf16(act_bf16, scratch_bf16, out_bf16, m, n, k, s), what);
}

int q2_0_prefill_gemm(const void *act_bf16, const void *w_q2, void *out_bf16, void *scratch_bf16,
                      void *act_q8, uint32_t m, uint32_t n, uint32_t k, uint32_t group, int use_mmq,
                      void *stream) {
  const bool mmq = use_mmq && group == 128u;
  const int st = check_prefill("q2_0_prefill_gemm", act_bf16, w_q2, out_bf16, scratch_bf16, act_q8, m, n, k,
                               group, mmq);
  if (st != BQ_OK) return st;
  return launch_prefill("q2_0_prefill_gemm", act_bf16, w_q2, out_bf16, scratch_bf16, act_q8, m, n, k, group,
                        mmq, as_stream(stream));
}

}  // extern "C"

// ---- the prefill dispatcher without a workspace argument ------------------
//
// Its workspace is this file-scope device array: every GPU the library runs
// on holds one copy, allocated when the library's code object is loaded there
// and kept until the process ends.  In host code the name `scratch` stands
// for the host-side shadow of the variable, not a device address; the
// device address is looked up once per device (scratch_address) and only
// that address is ever handed to kernels.
namespace {

constexpr uint64_t kScratchBytes = 64ull << 20;
constexpr uintptr_t kScratchAlign = 256;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

// Device address of `scratch` on the current device, looked up with that
// device current on its first use and remembered per device.
hipError_t scratch_address(void **ptr) {
  static std::mutex mu;
  static std::vector<std::pair<int, void *>> known;  // device, address
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  for (const auto &p : known)
    if (p.first == dev) {
      *ptr = p.second;
      return hipSuccess;
    }
  void *addr = nullptr;
  e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (addr == nullptr) return hipErrorInvalidSymbol;
  known.emplace_back(dev, addr);
  *ptr = addr;
  return hipSuccess;
}

}  // namespace

extern "C" {

int q2_0_prefill_gemm_noalloc(const void *act_bf16, const void *w_q2, void *out_bf16, uint32_t m, uint32_t n,
                              uint32_t k, uint32_t group, int use_mmq, void *stream) {
  const char *name = "q2_0_prefill_gemm_noalloc";
  const bool mmq = use_mmq && group == 128u;
  // The workspace the branch needs must fit the array.  The shared argument
  // checks then run with a stand-in workspace address (non-null, aligned,
  // below every caller buffer) so that, as for every call, a rejected call
  // makes no HIP call; the array's real address is looked up after them.
  const uint64_t need = mmq ? q8_bytes(m, k) : bf16_bytes(n, k);
  REQUIRE(need <= kScratchBytes, BQ_EUNSUPPORTED,
          "%s: the %s needs %llu bytes of workspace, more than the %llu this entry point holds "
          "(use q2_0_prefill_gemm with a caller buffer)",
          name, mmq ? "q8_1 activation buffer" : "bf16 dequant buffer", (unsigned long long)need,
          (unsigned long long)kScratchBytes);
  void *const stand_in = reinterpret_cast<void *>(uintptr_t{kScratchAlign});
  int st = check_prefill(name, act_bf16, w_q2, out_bf16, mmq ? nullptr : stand_in, mmq ? stand_in : nullptr,
                         m, n, k, group, mmq);
  if (st != BQ_OK) return st;
  void *ws = nullptr;
  st = hip_status(scratch_address(&ws), "q2_0_prefill_gemm_noalloc (workspace address)");
  if (st != BQ_OK) return st;
  return launch_prefill(name, act_bf16, w_q2, out_bf16, mmq ? nullptr : ws, mmq ? ws : nullptr, m, n, k, group,
                        mmq, as_stream(stream));
}

int silu_mul_bf16(const void *gate, const void *up, void *out, uint64_t count, void *stream) {
  REQUIRE(gate && up && out, BQ_EINVAL, "silu_mul_bf16: null pointer");
  REQUIRE(count >= 1, BQ_EINVAL, "silu_mul_bf16: count must be >= 1");
  REQUIRE(((reinterpret_cast<uintptr_t>(gate) | reinterpret_cast<uintptr_t>(up) |
            reinterpret_cast<uintptr_t>(out)) & 1u) == 0u,
          BQ_EALIGN, "silu_mul_bf16: bf16 buffers must be 2-byte aligned");
  REQUIRE(out == gate || !overlap(out, 2u * count, gate, 2u * count), BQ_EINVAL,
          "silu_mul_bf16: the output overlaps gate (only out == gate is allowed)");
  REQUIRE(!overlap(out, 2u * count, up, 2u * count), BQ_EINVAL, "silu_mul_bf16: the output overlaps up");
  return hip_status(bqmm::launch_silu_mul(gate, up, out, count, as_stream(stream)), "silu_mul_bf16");
}

}  // extern "C"

"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/bqmm.h declares, computes the buffer sizes, and
rejects bad arguments with the documented status before any HIP call."""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bqmm.h")


@pytest.fixture(scope="module")
def bq():
    import bit_quantized_matmul_quantize_amd as bq
    if not os.path.exists(bq.LIB_PATH):
        from bit_quantized_matmul_quantize_amd import build
        build.build()
    return bq


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z][a-z0-9_]*)\s*\(", text)) - {"if", "sizeof"})


def test_every_declared_symbol_is_exported(bq):
    names = declared_functions()
    assert len(names) >= 16, names
    l = bq.lib()
    for name in names:
        assert hasattr(l, name), name
    assert set(names) == set(bq.EXPORTS), set(names) ^ set(bq.EXPORTS)


def test_sizes_match_the_oracle_and_the_pages(bq):
    for m, k in [(1, 1), (4, 512), (3, 300), (2048, 2048), (4096, 17408)]:
        assert bq.q8_1_act_bytes(m, k) == oracle.q8_1_bytes(m, k)
    for n, k, g in [(256, 512, 128), (12288, 2048, 128), (5, 96, 32), (3, 512, 256)]:
        assert bq.q2_0_weight_bytes(n, k, g) == oracle.q2_0_bytes(n, k, g)
    assert bq.q2_0_weight_bytes(4, 100, 32) == 0 and bq.q2_0_weight_bytes(4, 96, 48) == 0
    # page layers/ops/q4k_mmq.rs, fn q4k_weight_bytes: nrows * (n_per_row / 256) * 144
    assert bq.q4k_weight_bytes(17408, 5120) == 17408 * 20 * 144
    assert bq.q4k_weight_bytes(4, 300) == 0


P = ctypes.c_void_p
A = P(0x10000)          # aligned fake device addresses: never dereferenced,
B = P(0x20000)          # every case below fails validation first
C = P(0x30000)
D = P(0x40000)
MIS = P(0x30008)        # misaligned


def _err(bq):
    return bq.lib().bq_last_error().decode()


@pytest.mark.parametrize("call,status,needle", [
    (lambda l: l.quantize_act_q8_1(None, B, 4, 512, None), -1, "null"),
    (lambda l: l.quantize_act_q8_1(A, B, 0, 512, None), -1, "m=0"),
    (lambda l: l.quantize_act_q8_1(A, MIS, 4, 512, None), -3, "aligned"),
    (lambda l: l.silu_mul_quantize_q8_1(A, None, C, 4, 512, None), -1, "null"),
    (lambda l: l.silu_mul_quantize_q8_1(A, MIS, C, 4, 512, None), -3, "aligned"),
    (lambda l: l.silu_mul_quantize_q8_1(A, B, C, 4, 0, None), -1, "k=0"),
    (lambda l: l.q2_0_mmq_gemm(A, B, C, 4, 256, 500, None), -1, "multiple of 128"),
    (lambda l: l.q2_0_mmq_gemm(A, B, C, 0, 256, 512, None), -1, "m=0"),
    (lambda l: l.q2_0_mmq_gemm(A, MIS, C, 4, 256, 512, None), -3, "aligned"),
    (lambda l: l.q2_0_mmq_gemm(A, B, C, 128 * 65536, 256, 512, None), -1, "too large"),
    (lambda l: l.q2_0_mmq_gemm_ldc(A, B, C, 4, 256, 512, 255, None), -1, "ldc=255"),
    (lambda l: l.q2_0_mmq_gemm_ldc(A, B, MIS, 4, 256, 512, 512, None), -3, "aligned"),
    (lambda l: l.q4k_mmq_gemm_ldc(A, B, C, 4, 256, 512, 100, None), -1, "ldc=100"),
    (lambda l: l.q2_0_gemv_vec(A, B, C, 256, 200, None), -1, "group size 128"),
    (lambda l: l.q2_0_gemv_vec(A, B, None, 256, 512, None), -1, "null"),
    (lambda l: l.q2_0_gemv_vec_batchm(A, B, C, 9, 256, 512, None), -2, "m=9"),
    (lambda l: l.q2_0_gemv_vec_batchm(A, B, C, 0, 256, 512, None), -1, "m must"),
    (lambda l: l.q2_0_gemv_gate_up_silu(A, B, C, D, 9, 256, 512, None), -2, "m=9"),
    (lambda l: l.q2_0_gemv_gate_up_silu(A, B, None, D, 2, 256, 512, None), -1, "null"),
    (lambda l: l.q2_0_gemv_gate_up_silu(A, B, MIS, D, 2, 256, 512, None), -3, "aligned"),
    (lambda l: l.q2_0_gemv_gate_up_silu(A, B, C, A, 2, 256, 512, None), -1, "overlaps the activations"),
    (lambda l: l.q2_0_gemv_gate_up_silu(A, B, C, P(0x30000 + 512), 2, 256, 512, None), -1, "overlaps the up weight"),
    (lambda l: l.q2_0_gemv_gate_up_silu(A, B, C, D, 2, 256, 300, None), -1, "group size 128"),
    (lambda l: l.dequant_q2_0_to_bf16(A, B, 4, 512, 48, None), -2, "multiple of 32"),
    (lambda l: l.dequant_q2_0_to_bf16(A, B, 4, 480, 128, None), -1, "not a multiple"),
    (lambda l: l.dense_gemm_bf16(A, B, C, 4, 4, 96, None), -1, "multiple of 64"),
    (lambda l: l.dense_gemm_bf16(A, B, C, 4, 128 * 65536, 64, None), -1, "too large"),
    (lambda l: l.q4k_mmq_gemm(A, B, C, 4, 4, 384, None), -1, "multiple of 256"),
    (lambda l: l.q2_0_prefill_gemm(A, B, C, None, None, 4, 4, 512, 128, 1, None), -1, "act_q8"),
    (lambda l: l.q2_0_prefill_gemm(A, B, C, None, None, 4, 4, 512, 128, 0, None), -1, "scratch"),
    (lambda l: l.q2_0_prefill_gemm(A, B, C, None, None, 4, 4, 512, 64, 1, None), -1, "scratch"),
    (lambda l: l.q2_0_prefill_gemm_noalloc(A, B, C, 4096, 64, 16384, 128, 1, None), -2, "workspace"),
    (lambda l: l.q2_0_prefill_gemm_noalloc(A, B, C, 4, 8192, 8192, 128, 0, None), -2, "workspace"),
    (lambda l: l.q2_0_prefill_gemm_noalloc(None, B, C, 4, 4, 512, 128, 1, None), -1, "null"),
    (lambda l: l.q2_0_prefill_gemm_noalloc(A, B, C, 4, 4, 500, 128, 1, None), -1, "multiple of 128"),
    (lambda l: l.q2_0_prefill_gemm_noalloc(A, B, C, 4, 4, 480, 64, 0, None), -1, "not a multiple"),
    (lambda l: l.q2_0_prefill_gemm_noalloc(A, B, P(0x20000 + 64), 4, 4, 512, 128, 1, None), -1, "overlaps the weight"),
    (lambda l: l.silu_mul_bf16(A, B, C, 0, None), -1, "count"),
    (lambda l: l.silu_mul_bf16(A, B, P(0x30001), 8, None), -3, "aligned"),
    (lambda l: l.q2_0_mmq_blockdots(A, B, C, 4, 1, 0, 1, 4, 256, 512, None), -1, "outside"),
    (lambda l: l.q2_0_mmq_blockdots(A, B, C, 0, 0, 0, 1, 4, 256, 512, None), -1, "empty"),
    (lambda l: l.q4k_mmq_blockdots(A, B, C, 0, 1, 250, 7, 4, 256, 512, None), -1, "outside"),
    (lambda l: l.q4k_gemv_vec(A, B, C, 256, 384, None), -1, "multiple of 256"),
    (lambda l: l.q4k_gemv_vec(A, B, C, 0, 512, None), -1, "n=0"),
    (lambda l: l.q4k_gemv_vec(None, B, C, 4, 512, None), -1, "null"),
    (lambda l: l.q4k_gemv_vec(A, MIS, C, 4, 512, None), -3, "aligned"),
    (lambda l: l.q4k_gemv_vec(A, B, C, 4, (1 << 30) + 256, None), -1, "too large"),
    (lambda l: l.quantize_weight_q4k(A, B, 4, 300, None), -1, "multiple of 256"),
    (lambda l: l.quantize_weight_q4k(A, None, 4, 512, None), -1, "null"),
    (lambda l: l.quantize_weight_q4k(A, MIS, 4, 512, None), -3, "aligned"),
    (lambda l: l.quantize_weight_q4k(A, B, 0, 512, None), -1, "n=0"),
    # sizes whose tile counts or padded row lengths would not fit 32 bits
    (lambda l: l.q2_0_mmq_gemm(A, B, C, 0xFFFFFFFF, 256, 512, None), -1, "too large"),
    (lambda l: l.q2_0_mmq_gemm(A, B, C, 4, 256, (1 << 30) + 128, None), -1, "too large"),
    (lambda l: l.q4k_mmq_gemm(A, B, C, 4, (1 << 31) + 1, 512, None), -1, "too large"),
    (lambda l: l.quantize_act_q8_1(A, B, 4, (1 << 30) + 1, None), -1, "too large"),
    (lambda l: l.silu_mul_quantize_q8_1(A, B, C, 4, 0xFFFFFFFF, None), -1, "too large"),
    (lambda l: l.q2_0_gemv_vec(A, B, C, 256, (1 << 30) + 128, None), -1, "too large"),
    (lambda l: l.q2_0_gemv_vec(A, B, C, (1 << 31) + 1, 512, None), -1, "too large"),
    (lambda l: l.q4k_gemv_vec(A, B, C, (1 << 31) + 1, 512, None), -1, "too large"),
    (lambda l: l.quantize_weight_q4k(A, B, 1 << 30, 1 << 20, None), -1, "too large"),
    (lambda l: l.dequant_q2_0_to_bf16(A, B, 4, (1 << 30) + 128, 128, None), -1, "too large"),
    (lambda l: l.dense_gemm_bf16(A, B, C, 4, 0xFFFFFFFF, 64, None), -1, "too large"),
    (lambda l: l.dense_gemm_bf16(A, B, C, (1 << 31) + 1, 4, 64, None), -1, "too large"),
    # outputs overlapping inputs (byte extents from the shapes)
    (lambda l: l.quantize_act_q8_1(A, P(0x10000 + 1024), 4, 512, None), -1, "overlaps the input"),
    (lambda l: l.silu_mul_quantize_q8_1(A, B, P(0x20000 + 16), 4, 512, None), -1, "overlaps up"),
    (lambda l: l.q2_0_mmq_gemm(A, B, P(0x20000 + 256), 4, 256, 512, None), -1, "overlaps the weight"),
    (lambda l: l.q2_0_mmq_gemm(A, B, A, 4, 256, 512, None), -1, "overlaps the q8_1"),
    # the row stride widens the written span: [m][n] alone would end before the weight
    (lambda l: l.q2_0_mmq_gemm_ldc(A, B, P(0x20000 - 4096), 4, 256, 512, 1024, None), -1, "overlaps the weight"),
    (lambda l: l.q4k_mmq_blockdots(A, B, P(0x20000 + 64), 0, 1, 0, 1, 4, 256, 512, None), -1, "overlaps the weight"),
    (lambda l: l.q2_0_gemv_vec(A, B, A, 256, 512, None), -1, "overlaps the activations"),
    (lambda l: l.q2_0_gemv_vec_batchm(A, B, P(0x20000 + 32), 3, 256, 512, None), -1, "overlaps the weight"),
    (lambda l: l.q4k_gemv_vec(A, B, B, 256, 512, None), -1, "overlaps the weight"),
    (lambda l: l.quantize_weight_q4k(A, A, 4, 512, None), -1, "overlaps the input"),
    (lambda l: l.dequant_q2_0_to_bf16(A, P(0x10000 + 64), 4, 512, 128, None), -1, "overlaps the weight"),
    (lambda l: l.dense_gemm_bf16(A, B, P(0x20000 + 128), 4, 4, 64, None), -1, "overlaps the weight"),
    (lambda l: l.q2_0_prefill_gemm(A, B, C, None, P(0x10000 + 64), 4, 4, 512, 128, 1, None), -1, "overlaps the input"),
    (lambda l: l.q2_0_prefill_gemm(A, B, C, P(0x10000 + 64), None, 4, 4, 512, 128, 0, None), -1, "overlaps the input"),
    (lambda l: l.silu_mul_bf16(A, B, P(0x10000 + 16), 64, None), -1, "overlaps gate"),
    (lambda l: l.silu_mul_bf16(A, B, B, 64, None), -1, "overlaps up"),
])
def test_validation_rejects_before_any_hip_call(bq, call, status, needle):
    assert call(bq.lib()) == status
    assert needle in _err(bq), _err(bq)


def test_status_strings(bq):
    l = bq.lib()
    assert l.bq_status_string(0) == b"ok"
    assert l.bq_status_string(-2) == b"unsupported configuration"
    assert l.bq_status_string(7) == b"unknown status"


def test_python_binding_raises_on_bad_status(bq):
    with pytest.raises(bq.BqmmError) as e:
        bq._check(bq.lib().q2_0_gemv_vec_batchm(A, B, C, 9, 256, 512, None))
    assert e.value.status == bq.BQ_EUNSUPPORTED

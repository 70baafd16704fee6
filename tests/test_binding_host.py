"""Host-side checks of the Python binding (no GPU): every wrapper rejects a
tensor smaller than the bytes its shape arguments address, a wrong dtype, and
host tensors, before anything reaches the library's kernels."""
import pytest
import torch


@pytest.fixture(scope="module")
def bq():
    import os
    import bit_quantized_matmul_quantize_amd as m
    if not os.path.exists(m.LIB_PATH):
        from bit_quantized_matmul_quantize_amd import build
        build.build()
    return m


def bf(n):
    return torch.zeros(n, dtype=torch.bfloat16)


def u8(n):
    return torch.zeros(n, dtype=torch.uint8)


M, N, K = 4, 256, 512


def _cases(bq):
    q8 = bq.q8_1_act_bytes(M, K)
    q2 = bq.q2_0_weight_bytes(N, K)
    q4 = bq.q4k_weight_bytes(N, K)
    # (call with one buffer one byte/element short, its name)
    return [
        (lambda: bq.quantize_act_q8_1(bf(M * K - 1), u8(q8), M, K), "act"),
        (lambda: bq.quantize_act_q8_1(bf(M * K), u8(q8 - 1), M, K), "out_q8"),
        (lambda: bq.silu_mul_quantize_q8_1(bf(M * K), bf(M * K - 1), u8(q8), M, K), "up"),
        (lambda: bq.q2_0_mmq_gemm(u8(q8), u8(q2 - 1), bf(M * N), M, N, K), "w_q2"),
        (lambda: bq.q2_0_mmq_gemm(u8(q8), u8(q2), bf(M * N - 1), M, N, K), "out"),
        (lambda: bq.q2_0_mmq_gemm_ldc(u8(q8 - 1), u8(q2), bf(M * N).view(M, N), M, N, K, N), "act_q8"),
        (lambda: bq.q4k_mmq_gemm(u8(q8), u8(q4 - 1), bf(M * N), M, N, K), "w_q4k"),
        (lambda: bq.q4k_mmq_gemm_ldc(u8(q8), u8(q4 - 1), bf(M * N).view(M, N), M, N, K, N), "w_q4k"),
        (lambda: bq.q2_0_gemv_vec(bf(K - 1), u8(q2), bf(N), N, K), "act"),
        (lambda: bq.q2_0_gemv_vec_batchm(bf(3 * K), u8(q2), bf(3 * N - 1), 3, N, K), "out"),
        (lambda: bq.q2_0_gemv_gate_up_silu(bf(2 * K), u8(q2), u8(q2 - 1), bf(2 * N), 2, N, K), "w_up"),
        (lambda: bq.dequant_q2_0_to_bf16(u8(q2), bf(N * K - 1), N, K), "out"),
        (lambda: bq.dense_gemm_bf16(bf(M * K), bf(N * K - 1), bf(M * N), M, N, K), "w"),
        (lambda: bq.q2_0_prefill_gemm(bf(M * K), u8(q2), bf(M * N), None, u8(q8 - 1), M, N, K), "act_q8"),
        (lambda: bq.q2_0_prefill_gemm(bf(M * K), u8(q2), bf(M * N), bf(N * K - 1), None, M, N, K,
                                      use_mmq=False), "scratch"),
        (lambda: bq.q4k_gemv_vec(bf(K), u8(q4), bf(N - 1), N, K), "out"),
        (lambda: bq.quantize_weight_q4k(bf(N * K), u8(q4 - 1), N, K), "out_q4k"),
        (lambda: bq.silu_mul_bf16(bf(64), bf(63), bf(64), 64), "up"),
        (lambda: bq.q2_0_mmq_blockdots(u8(q8), u8(q2), torch.zeros(4 * 4 * (K // 32) - 1, dtype=torch.int32),
                                       0, 4, 0, 4, M, N, K), "out_i32"),
    ]


def test_every_short_buffer_is_rejected(bq):
    for call, what in _cases(bq):
        with pytest.raises(ValueError) as e:
            call()
        assert str(e.value).startswith(what + ":") and "address" in str(e.value), str(e.value)


def test_full_size_host_tensors_are_rejected(bq):
    q2 = bq.q2_0_weight_bytes(N, K)
    with pytest.raises(ValueError, match="device tensor"):
        bq.q2_0_gemv_vec(bf(K), u8(q2), bf(N), N, K)


def test_dtypes_are_checked(bq):
    q2 = bq.q2_0_weight_bytes(N, K)
    with pytest.raises(TypeError, match="bfloat16"):
        bq.q2_0_gemv_vec(torch.zeros(K, dtype=torch.float32), u8(q2), bf(N), N, K)
    with pytest.raises(TypeError, match="uint8"):
        bq.q2_0_gemv_vec(bf(K), bf(q2), bf(N), N, K)
    with pytest.raises(TypeError, match="int32"):
        bq.q2_0_mmq_blockdots(u8(bq.q8_1_act_bytes(M, K)), u8(q2), u8(4096), 0, 1, 0, 1, M, N, K)


def test_strided_output_view_passes_the_binding_checks(bq):
    # a column range of a wider buffer is a valid output for the _ldc calls:
    # host tensors get as far as the device check
    q8, q2 = bq.q8_1_act_bytes(M, K), bq.q2_0_weight_bytes(N, K)
    big = bf(M * (N + 64)).view(M, N + 64)
    with pytest.raises(ValueError, match="device tensor"):
        bq.q2_0_mmq_gemm_ldc(u8(q8), u8(q2), big[:, 8:8 + N], M, N, K, N + 64)

"""GPU parity: the Q4_K decode GEMV (floats within the row-L2 bound) and the
Q4_K weight quantizer (bytes bit-exact), through the C ABI, against the
oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import inputs
import oracle
import bit_quantized_matmul_quantize_amd as bq
from parity_helpers import (ROW_TOL, bf16_ulp_distance, dev_bf16, dev_u8, empty_bf16, host_bits, host_f64,
                            rows_ok, row_error)

pytestmark = pytest.mark.gpu


def _gemv(gpu, a, w, n, k):
    out = empty_bf16((n,), gpu)
    bq.q4k_gemv_vec(dev_bf16(a, gpu), dev_u8(w, gpu), out, n, k)
    return out


# --- decode GEMV -----------------------------------------------------------

# FFN gate/up [17408, 5120] and down [5120, 17408] at full size; ragged row
# counts (the last workgroup partly filled), unit counts that leave a ragged
# last slice of 16 (k = 768, 4352), the smallest and largest k.
@pytest.mark.parametrize("n,k,seed", [(17408, 5120, 101), (5120, 17408, 102), (16385, 2048, 103),
                                      (1000, 4352, 104), (256, 1024, 105)])
def test_gemv_workload_shapes(gpu, n, k, seed):
    g = inputs.rng(seed)
    w = inputs.q4k_weight(g, n, k)
    a = inputs.activations(g, 1, k, outliers=True)
    y = host_f64(_gemv(gpu, a, w, n, k))
    R = oracle.q4k_gemv(a, w, 1, n, k)[0]
    print(f"q4k_gemv n={n} k={k}: row error {row_error(y, R):.2e}", flush=True)
    assert row_error(y, R) <= ROW_TOL


@pytest.mark.parametrize("n,k,seed", [(7, 512, 111), (33, 768, 112), (1, 256, 113), (3, 256, 114),
                                      (64, 65536, 115), (17, 1280, 116),
                                      # past one LDS chunk of 65536 values: a second, ragged
                                      # chunk, and three full chunks
                                      (9, 65536 + 1280, 119), (5, 3 * 65536, 120)])
def test_gemv_edge_shapes(gpu, n, k, seed):
    g = inputs.rng(seed)
    w = inputs.q4k_weight(g, n, k)
    a = inputs.activations(g, 1, k, outliers=True)
    y = host_f64(_gemv(gpu, a, w, n, k))
    R = oracle.q4k_gemv(a, w, 1, n, k)[0]
    assert rows_ok(y, R)


def test_gemv_zero_activations(gpu):
    n, k = 300, 1024
    w = inputs.q4k_weight(inputs.rng(117), n, k)
    a = np.zeros((1, k), np.uint16)
    assert not np.any(host_f64(_gemv(gpu, a, w, n, k)))


def test_gemv_one_hot_columns(gpu):
    """A one-hot activation returns one weight column: the dequantized value,
    rounded once to fp32 and once to bf16 (at most one bf16 step from the
    fp64 value rounded to bf16)."""
    n, k = 96, 768
    w = inputs.q4k_weight(inputs.rng(118), n, k)
    for col in (0, 31, 32, 63, 64, 200, 511, 767):
        a = np.zeros((1, k), np.uint16)
        a[0, col] = 0x3F80
        R = oracle.q4k_gemv(a, w, 1, n, k)[0]
        got = host_bits(_gemv(gpu, a, w, n, k))
        assert bf16_ulp_distance(got, oracle.round_bf16(R)).max() <= 1, col


def test_gemv_rejects(gpu):
    a = torch.zeros(512, dtype=torch.bfloat16, device=gpu)
    w = torch.zeros(oracle.q4k_bytes(4, 512), dtype=torch.uint8, device=gpu)
    out = empty_bf16((4,), gpu)
    with pytest.raises(bq.BqmmError):
        bq.q4k_gemv_vec(a, w, out, 4, 500)


# --- weight quantizer ------------------------------------------------------

def _quantize(gpu, x_bits, n, k):
    out = torch.empty(oracle.q4k_bytes(n, k), dtype=torch.uint8, device=gpu)
    bq.quantize_weight_q4k(dev_bf16(x_bits, gpu), out, n, k)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _weights(seed, n, k, scale):
    g = inputs.rng(seed)
    x = g.standard_normal((n, k)).astype(np.float32) * scale
    if n >= 4 and k >= 512:
        x[0, 0:32] = np.abs(x[0, 0:32]) + scale       # all positive sub-block
        x[0, 32:64] = -np.abs(x[0, 32:64]) - scale    # all negative
        x[1, 0:32] = 0.5 * scale                      # constant
        x[1, 64:96] = 0.0                             # zeros
        x[2, 300] = 40 * scale                        # outlier
        x[3, 256:512] = 0.0                           # zero super-block
    bits = inputs.f32_to_bf16_bits(x)
    if n >= 4 and k >= 512:
        bits[3, 256:320] = 0x8000                     # negative zeros
    return bits


@pytest.mark.parametrize("n,k,seed,scale", [(64, 1024, 121, 0.02), (3, 768, 122, 1.0), (1, 256, 123, 0.02),
                                            (37, 2304, 124, 1e-6), (8, 512, 125, 300.0)])
def test_quantize_bit_exact(gpu, n, k, seed, scale):
    x = _weights(seed, n, k, scale)
    ref, flagged = oracle.quantize_weight_q4k(x, n, k)
    assert flagged == 0
    assert np.array_equal(_quantize(gpu, x, n, k), ref)


def test_quantize_full_size_bit_exact(gpu):
    n, k = 17408, 5120
    x = _weights(126, n, k, 0.02)
    ref, flagged = oracle.quantize_weight_q4k(x, n, k)
    assert flagged == 0
    got = _quantize(gpu, x, n, k)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:4]}"


def test_quantize_then_gemv(gpu):
    """Weights quantized on the device feed the decode GEMV; the result meets
    the bound against the oracle's GEMV over the oracle's own quantization."""
    n, k = 512, 2048
    x = _weights(127, n, k, 0.02)
    w_ref, _ = oracle.quantize_weight_q4k(x, n, k)
    wq = torch.empty(oracle.q4k_bytes(n, k), dtype=torch.uint8, device=gpu)
    bq.quantize_weight_q4k(dev_bf16(x, gpu), wq, n, k)
    a = inputs.activations(inputs.rng(128), 1, k)
    out = empty_bf16((n,), gpu)
    bq.q4k_gemv_vec(dev_bf16(a, gpu), wq, out, n, k)
    R = oracle.q4k_gemv(a, w_ref, 1, n, k)[0]
    assert row_error(host_f64(out), R) <= ROW_TOL


def test_quantize_near_ties(gpu):
    """Super-blocks whose sub-scale, sub-min and code quotients sit exactly on
    halves (the CPU pin's tie block, scaled by powers of two so the ties stay
    exact) and copies with about a third of their nonzero values moved one
    bf16 step up or down (quotients just off the halves): the device bytes
    equal the oracle's."""
    from test_oracle_q4k_gemv_quant import _tie_block
    tie_bits, _ = _tie_block()
    tie = inputs.bf16_bits_to_f32(tie_bits)
    g = inputs.rng(129)
    blocks = []
    for s in range(-1, 15):  # d = 2^(s - 13): binary16 normal throughout
        exact = inputs.f32_to_bf16_bits(tie * np.float32(2.0 ** s))
        blocks.append(exact)
        for _ in range(3):
            pick = (g.random(256) < 0.3) & ((exact & 0x7FFF) != 0)
            step = g.choice(np.array([-1, 1], np.int32), size=256)
            blocks.append(np.where(pick, (exact.astype(np.int32) + step).astype(np.uint16), exact))
    n, k = len(blocks) // 4, 1024  # 16 rows of 4 super-blocks
    x = np.stack(blocks).reshape(n, k)
    ref, flagged = oracle.quantize_weight_q4k(x, n, k)
    assert flagged == 0
    assert np.array_equal(_quantize(gpu, x, n, k), ref)

"""GPU parity: Q2_0 GEMV (m = 1), batched GEMV (m = 2..8), silu_mul and the
verify-batch FFN chain gate -> up -> silu_mul -> down."""
import numpy as np
import pytest
import torch

import inputs
import oracle
import bit_quantized_matmul_quantize_amd as bq
from parity_helpers import (ROW_TOL, bf16_ulp_distance, dev_bf16, dev_u8, empty_bf16, host_bits, host_f64,
                            rows_ok, row_error)

pytestmark = pytest.mark.gpu


def _gemv(gpu, act, w, m, n, k):
    out = empty_bf16((m, n), gpu)
    if m == 1:
        bq.q2_0_gemv_vec(dev_bf16(act, gpu), dev_u8(w, gpu), out, n, k)
    else:
        bq.q2_0_gemv_vec_batchm(dev_bf16(act, gpu), dev_u8(w, gpu), out, m, n, k)
    return host_f64(out)


def test_tiny_row0(gpu):
    d = inputs.tiny()
    act = d["act"][:1]
    R = oracle.q2_0_gemv(act, d["w"], 1, d["n"], d["k"])
    assert row_error(_gemv(gpu, act, d["w"], 1, d["n"], d["k"]), R) <= ROW_TOL


def test_decode_qkvz_full(gpu):
    d = inputs.decode_gemv()
    R = oracle.q2_0_gemv(d["act"], d["w"], 1, d["n"], d["k"])
    assert row_error(_gemv(gpu, d["act"], d["w"], 1, d["n"], d["k"]), R) <= ROW_TOL


@pytest.mark.parametrize("m,n,k,seed", [(1, 1, 128, 21), (1, 17, 384, 22), (3, 300, 1152, 23),
                                        (8, 33, 5120, 24), (5, 7, 17408, 25),
                                        (1, 50, 5120, 29),      # m=1: three 32-chunk slices, ragged last
                                        (1, 100, 17408, 30),    # m=1: prep loop over 1088 items
                                        (1, 3, 33792, 31),      # m=1 beyond the LDS-staged kernel's k
                                        (1, 4096 + 37, 2048, 32),
                                        # m = 2, 3 on wide outputs (n >= 8192; m = 3 on matrix cores):
                                        (2, 8192 + 45, 1152, 33),   # two slices, the second ragged
                                        (3, 9000, 384, 34),         # one slice, fewer than the prefetch depth
                                        (3, 8192, 4096, 35),        # one full prefetch round plus one slice
                                        (1, 8192 + 5, 36864, 36),   # m=1 beyond the decode kernel's k
                                        (4, 9, 65536 + 1024, 37),   # m >= 3 beyond the matrix-core kernel's k
                                        # matrix-core kernel (m >= 3): one wave per group range
                                        (6, 100, 512, 39), (6, 8192 + 16, 2048, 40),
                                        (4, 8192 + 16, 2048, 41),   # wide: 3 tiles per wave, last workgroup ragged
                                        (5, 1000, 1024, 42),        # narrow: 2 tiles per wave, ragged
                                        (4, 151, 1152, 43),
                                        # whole-vector kernel (m = 1, 2): shortest k, and the largest
                                        # k whose activations fit its LDS for each m, and one past it
                                        # (m = 3 at those shapes runs on the matrix-core kernel)
                                        (2, 5, 128, 44), (3, 49, 256, 45), (1, 77, 28672, 46),
                                        (2, 65, 13312, 47), (3, 33, 9216, 48), (2, 33, 13440, 49),
                                        (1, 4096 + 16, 4096, 50),
                                        # whole-vector kernel, m = 1 with three weight register sets
                                        # (k >= 12288): 12 chunks per lane, and 13 with a ragged last
                                        (1, 41, 12288, 51), (1, 29, 12416, 52),
                                        # m=1 decode kernel with more than 64 KB of staged activations
                                        # (k past the whole-vector kernel's LDS, up to its own limit)
                                        (1, 300, 30720, 53), (1, 17, 32768, 54),
                                        # m >= 3: the largest k of the matrix-core kernel, and one group
                                        # past it (the vector kernel)
                                        (4, 300, 37888, 55), (5, 40, 38016, 56), (4, 33, 49152, 57),
                                        (3, 40, 37888, 66), (3, 40, 38016, 67),
                                        # m >= 3, balanced rows (one workgroup per compute unit, used
                                        # where the plain grid has more workgroups than units): 4, 5
                                        # and 6 tiles per workgroup, the last tile overlapping the one
                                        # before it, the last workgroup ragged; then past six tiles
                                        # (the plain launch in more than one round)
                                        (4, 12288 + 1, 1152, 58), (8, 16384 + 77, 1024, 59),
                                        (5, 20480 + 1, 1152, 60), (6, 24576, 1024, 61),
                                        (7, 24576 + 100, 1152, 62),
                                        # m >= 3 with one wave (fewer than eight groups): one group
                                        # (its pair load reads the group twice), two, and three (a
                                        # pair and a single group)
                                        (4, 20, 128, 63), (5, 17, 256, 64), (8, 9, 384, 65),
                                        (3, 20, 128, 68), (3, 12288 + 1, 1152, 69)])
def test_ragged(gpu, m, n, k, seed):
    g = inputs.rng(seed)
    w = inputs.q2_0_weight(g, n, k)
    act = inputs.activations(g, m, k, outliers=True)
    R = oracle.q2_0_gemv(act, w, m, n, k)
    assert rows_ok(_gemv(gpu, act, w, m, n, k), R)


def test_closed_forms(gpu):
    # codes 2 -> exactly 0; codes 3 with d = 1 -> row sums (exact for integer inputs)
    n, k = 5, 256
    g = inputs.rng(26)
    x = g.integers(-4, 5, size=(2, k)).astype(np.float32)
    act = inputs.f32_to_bf16_bits(x)
    ones = np.frombuffer(np.ones(n * 2, np.float16).tobytes(), np.uint8)
    w2 = np.concatenate([np.full(n * k // 4, 0xAA, np.uint8), ones])
    w3 = np.concatenate([np.full(n * k // 4, 0xFF, np.uint8), ones])
    assert not _gemv(gpu, act, w2, 2, n, k).any()
    y = _gemv(gpu, act, w3, 2, n, k)
    assert np.array_equal(y, np.repeat(x.sum(1, keepdims=True).astype(np.float64), n, axis=1))


@pytest.mark.parametrize("m,n,k", [(1, 300, 2048), (1, 64, 33792), (3, 640, 5120), (8, 8200, 1024)])
def test_zero_activations(gpu, m, n, k):
    # zero activations give exactly zero outputs (no bias residue)
    w = inputs.q2_0_weight(inputs.rng(37), n, k)
    act = np.zeros((m, k), np.uint16)
    assert not _gemv(gpu, act, w, m, n, k).any()


def test_sparse_activations(gpu):
    # a mostly-zero activation row (every 7th value kept) against the oracle
    m, n, k = 3, 700, 5120
    g = inputs.rng(38)
    w = inputs.q2_0_weight(g, n, k)
    act = inputs.activations(g, m, k)
    act[:, np.arange(k) % 7 != 0] = 0
    R = oracle.q2_0_gemv(act, w, m, n, k)
    assert row_error(_gemv(gpu, act, w, m, n, k), R) <= ROW_TOL


@pytest.mark.parametrize("m", [2, 5, 8])
def test_batch_rows_independent(gpu, m):
    # a row's output does not depend on the other rows of the batch: replacing
    # rows 1.. leaves row 0 bit-identical (same m, same kernel)
    n, k = 640, 2048
    g = inputs.rng(27)
    w = inputs.q2_0_weight(g, n, k)
    act = inputs.activations(g, m, k)
    other = act.copy()
    other[1:] = inputs.activations(g, m - 1, k)
    y = _gemv(gpu, act, w, m, n, k)
    y_other = _gemv(gpu, other, w, m, n, k)
    assert np.array_equal(y[0], y_other[0])
    assert row_error(y, oracle.q2_0_gemv(act, w, m, n, k)) <= ROW_TOL


def test_silu_mul(gpu):
    g = inputs.rng(28)
    for count in (1, 7, 8, 4097, 8 * 17408):
        gate = inputs.activations(g, 1, count)[0]
        up = inputs.activations(g, 1, count)[0]
        ref = oracle.silu_mul_bf16(gate, up)
        gd, ud = dev_bf16(gate, gpu), dev_bf16(up, gpu)
        out = empty_bf16((count,), gpu)
        bq.silu_mul_bf16(gd, ud, out)
        got = host_bits(out)
        # within one bf16 step (binary32 arithmetic on the device, fp64 in the oracle)
        assert bf16_ulp_distance(got, ref).max() <= 1
        # in place over the gate buffer gives the same bits
        bq.silu_mul_bf16(gd, ud, gd)
        assert np.array_equal(host_bits(gd), got)


def test_silu_mul_wide_gate_range(gpu):
    """Gate values from -87 to 100: exp(-g) reaches 6e37 at the low end and
    underflows at the high end; one bf16 step still holds there. Below about
    -87.3 the device result may be +-0: it stays under 1e-35 * |up|."""
    g = inputs.rng(29)
    count = 65536
    gate = np.array([oracle.f64_to_bf16(x) for x in np.linspace(-87.0, 100.0, count)],
                    dtype=np.uint16)
    up = inputs.activations(g, 1, count)[0]
    ref = oracle.silu_mul_bf16(gate, up)
    out = empty_bf16((count,), gpu)
    bq.silu_mul_bf16(dev_bf16(gate, gpu), dev_bf16(up, gpu), out)
    assert bf16_ulp_distance(host_bits(out), ref).max() <= 1
    low = np.array([oracle.f64_to_bf16(x) for x in (-88.0, -90.0, -200.0)], dtype=np.uint16)
    up3 = inputs.activations(g, 1, 3)[0]
    out3 = empty_bf16((3,), gpu)
    bq.silu_mul_bf16(dev_bf16(low, gpu), dev_bf16(up3, gpu), out3)
    got3 = inputs.bf16_bits_to_f32(host_bits(out3)).astype(np.float64)
    assert np.all(np.abs(got3) <= 1e-35 * np.abs(inputs.bf16_bits_to_f32(up3)))


@pytest.fixture(scope="module")
def ffn():
    return inputs.verify_ffn()


@pytest.mark.parametrize("m", [2, 3, 4, 8])
def test_verify_ffn_chain(gpu, ffn, m):
    H, I = ffn["hidden"], ffn["inter"]
    x = ffn["act"][:m]
    wg, wu, wdn = (dev_u8(ffn[key], gpu) for key in ("wg", "wu", "wd"))
    xd = dev_bf16(x, gpu)
    gate, up, out = empty_bf16((m, I), gpu), empty_bf16((m, I), gpu), empty_bf16((m, H), gpu)
    bq.q2_0_gemv_vec_batchm(xd, wg, gate, m, I, H)
    bq.q2_0_gemv_vec_batchm(xd, wu, up, m, I, H)
    g_bits, u_bits = host_bits(gate), host_bits(up)
    bq.silu_mul_bf16(gate, up, gate, m * I)
    h_bits = host_bits(gate)
    bq.q2_0_gemv_vec_batchm(gate, wdn, out, m, H, I)
    y = host_f64(out)
    # stage-wise: each stage against the oracle on the device's own previous output
    Rg = oracle.q2_0_gemv(x, ffn["wg"], m, I, H)
    Ru = oracle.q2_0_gemv(x, ffn["wu"], m, I, H)
    assert row_error(inputs.bf16_bits_to_f32(g_bits).astype(np.float64), Rg) <= ROW_TOL
    assert row_error(inputs.bf16_bits_to_f32(u_bits).astype(np.float64), Ru) <= ROW_TOL
    Rh = oracle.silu_mul_bf16(g_bits, u_bits)
    assert bf16_ulp_distance(h_bits, Rh).max() <= 1
    Rd = oracle.q2_0_gemv(h_bits, ffn["wd"], m, H, I)
    assert row_error(y, Rd) <= ROW_TOL
    # end to end against the oracle's own chain (rounded to bf16 at the same points)
    Rend = oracle.q2_0_gemv(oracle.silu_mul_bf16(oracle.round_bf16(Rg), oracle.round_bf16(Ru)),
                            ffn["wd"], m, H, I)
    assert row_error(y, Rend) <= ROW_TOL


# ---- fused gate/up GEMV with the SiLU-gated product ---------------------------

def _fused(gpu, act, wg, wu, m, n, k):
    out = empty_bf16((m, n), gpu)
    bq.q2_0_gemv_gate_up_silu(dev_bf16(act, gpu), dev_u8(wg, gpu), dev_u8(wu, gpu), out, m, n, k)
    return host_bits(out)


def _chain_bits(gpu, act, wg, wu, m, n, k):
    """GEMV, GEMV, silu_mul on the device: the calls the fused entry replaces."""
    x = dev_bf16(act, gpu)
    g, u = empty_bf16((m, n), gpu), empty_bf16((m, n), gpu)
    if m == 1:
        bq.q2_0_gemv_vec(x, dev_u8(wg, gpu), g, n, k)
        bq.q2_0_gemv_vec(x, dev_u8(wu, gpu), u, n, k)
    else:
        bq.q2_0_gemv_vec_batchm(x, dev_u8(wg, gpu), g, m, n, k)
        bq.q2_0_gemv_vec_batchm(x, dev_u8(wu, gpu), u, m, n, k)
    bq.silu_mul_bf16(g, u, g, m * n)
    return host_bits(g)


@pytest.mark.parametrize("m,n,k,seed", [(2, 17408, 5120, 41), (3, 300, 1152, 42), (5, 8192 + 45, 2048, 43),
                                        (4, 33, 17408, 44), (8, 17408, 5120, 46), (6, 300, 1152, 47),
                                        (7, 40, 512, 48), (3, 33, 9216, 49), (2, 5, 128, 50),
                                        # the matrix-core kernel's largest k, and the vector kernel past it
                                        (4, 40, 37888, 51), (4, 40, 49152, 52), (8, 20, 38016, 53),
                                        # balanced rows: four tiles for both kernels; then six tiles
                                        # for the single GEMV and the plain launch for the fused one
                                        (4, 12288 + 1, 1152, 54), (6, 20480 + 1, 1024, 55)])
def test_fused_gate_up_equals_chain(gpu, m, n, k, seed):
    # m >= 2: the fused kernel sums every row exactly as the single GEMV does
    # (same kernel family, lane-group width and chunk order for each m)
    g = inputs.rng(seed)
    wg, wu = inputs.q2_0_weight(g, n, k), inputs.q2_0_weight(g, n, k)
    act = inputs.activations(g, m, k, outliers=True)
    assert np.array_equal(_fused(gpu, act, wg, wu, m, n, k), _chain_bits(gpu, act, wg, wu, m, n, k))


@pytest.mark.parametrize("m", [1, 2, 3, 6, 8])
def test_fused_gate_up_ffn_chain(gpu, ffn, m):
    # the verify FFN with the fused first stage, end to end against the oracle's
    # chain (bf16 roundings at the same points)
    H, I = ffn["hidden"], ffn["inter"]
    x = ffn["act"][:m]
    h_bits = _fused(gpu, x, ffn["wg"], ffn["wu"], m, I, H)
    out = empty_bf16((m, H), gpu)
    bq.q2_0_gemv_vec_batchm(dev_bf16(h_bits, gpu), dev_u8(ffn["wd"], gpu), out, m, H, I) if m > 1 else \
        bq.q2_0_gemv_vec(dev_bf16(h_bits, gpu), dev_u8(ffn["wd"], gpu), out, H, I)
    y = host_f64(out)
    Rg = oracle.q2_0_gemv(x, ffn["wg"], m, I, H)
    Ru = oracle.q2_0_gemv(x, ffn["wu"], m, I, H)
    Rend = oracle.q2_0_gemv(oracle.silu_mul_bf16(oracle.round_bf16(Rg), oracle.round_bf16(Ru)),
                            ffn["wd"], m, H, I)
    assert row_error(y, Rend) <= ROW_TOL
    # the fused output itself, every element, at the row-normalised bound
    # against the oracle's chain with the bf16 roundings at the device's
    # points, silu(bf16(g)) * bf16(u) rounded to bf16
    Rh_bits = oracle.silu_mul_bf16(oracle.round_bf16(Rg), oracle.round_bf16(Ru))
    hx = inputs.bf16_bits_to_f32(h_bits).astype(np.float64)
    assert row_error(hx, inputs.bf16_bits_to_f32(Rh_bits).astype(np.float64)) <= ROW_TOL
    # and almost every value within one bf16 step of it (the rest are where g
    # or u rounded to a neighbouring bf16 value)
    assert np.mean(bf16_ulp_distance(h_bits, Rh_bits) <= 1) > 0.99


def test_fused_gate_up_zero_and_ragged(gpu):
    n, k = 37, 384
    g = inputs.rng(45)
    wg, wu = inputs.q2_0_weight(g, n, k), inputs.q2_0_weight(g, n, k)
    assert not inputs.bf16_bits_to_f32(_fused(gpu, np.zeros((3, k), np.uint16), wg, wu, 3, n, k)).any()

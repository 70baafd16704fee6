"""Pins of the oracle's Q2_0 routines: decode, bf16 dequant, block dots, MMQ,
GEMV, dense bf16 GEMM and silu_mul.

Pins used (none re-types the oracle's own code):
  * hand-packed bytes whose decoded values are worked out by hand from the
    adopted layout (byte t of a group holds k-offsets t + j*G/4 in bits 2j..2j+1),
  * an independent pure-Python unpacker (per-byte bit expansion) plus
    dequantize-then-fp64-matmul brute force on tiny shapes,
  * the identity linking the integer block dots to the plain result,
  * closed forms (all codes 2 -> 0; codes 3 with d = 1 -> row sums; one-hot
    weights pick one activation; integer activations give exact integers),
  * library routines: numpy's fp64 matmul, torch's bf16 rounding, libm exp.
"""
import numpy as np
import pytest
import torch

import inputs
import oracle


def _q2_weight(codes: np.ndarray, scales: np.ndarray, group: int) -> np.ndarray:
    """Independent packer from the layout text: codes [n][k] in 0..3, scales
    [n][k/G] float -> bytes."""
    n, k = codes.shape
    q = group // 4
    out = np.zeros((n, k // 4), dtype=np.uint8)
    for r in range(n):
        for g in range(k // group):
            for t in range(q):
                byte = 0
                for j in range(4):
                    byte |= int(codes[r, g * group + t + j * q]) << (2 * j)
                out[r, g * q + t] = byte
    return np.concatenate([out.reshape(-1), scales.astype(np.float16).reshape(-1).view(np.uint8)])


def _py_unpack(w: np.ndarray, n: int, k: int, group: int):
    """Independent unpacker: expand each byte's four 2-bit fields."""
    q = group // 4
    plane = w[: n * k // 4].reshape(n, k // group, q)
    fields = np.stack([(plane >> (2 * j)) & 3 for j in range(4)], axis=2)  # [n][G][j][t]
    codes = fields.reshape(n, k).astype(np.int64)
    scales = w[n * k // 4:].view(np.float16).astype(np.float64).reshape(n, k // group)
    return codes, scales


def test_size():
    # 2.125 bits per weight at group 128: n*k/4 code bytes + 2 bytes per group
    assert oracle.q2_0_bytes(12288, 2048) == 12288 * 2048 // 4 + 2 * 12288 * 16 == 6684672


def test_hand_bytes_e4():
    # Every byte 0xE4 = 0b11_10_01_00: fields j=0..3 hold codes 0, 1, 2, 3.
    # So k-offsets t, t+32, t+64, t+96 (t = 0..31) get codes 0, 1, 2, 3 and with
    # d = 0.5 the weights are -1, -0.5, 0, 0.5 in four runs of 32.
    w = np.concatenate([np.full(32, 0xE4, np.uint8), np.array([0.5], np.float16).view(np.uint8)])
    dec = oracle.q2_0_decode(w, 1, 128)[0]
    assert dec.tolist() == [-1.0] * 32 + [-0.5] * 32 + [0.0] * 32 + [0.5] * 32


def test_hand_bytes_single_fields():
    # 0xAA = codes 2,2,2,2 -> all zero.  Byte 5 = 0xAB sets field j=0 to 3 -> only
    # k = 5 is +d.  Byte 7 = 0x2A sets field j=3 to 0 -> k = 7 + 96 = 103 is -2d.
    base = np.full(32, 0xAA, np.uint8)
    base[5] = 0xAB
    base[7] = 0x2A
    w = np.concatenate([base, np.array([0.25], np.float16).view(np.uint8)])
    dec = oracle.q2_0_decode(w, 1, 128)[0]
    expect = np.zeros(128)
    expect[5] = 0.25
    expect[103] = -0.5
    assert np.array_equal(dec, expect)


def test_scale_plane_order():
    # 2 rows x 2 groups, all codes 3 (w = d), scales row-major [row][group].
    codes = np.full((2, 256), 3)
    sc = np.array([[1.0, 2.0], [4.0, 8.0]])
    w = _q2_weight(codes, sc, 128)
    dec = oracle.q2_0_decode(w, 2, 256)
    assert np.all(dec[0, :128] == 1) and np.all(dec[0, 128:] == 2)
    assert np.all(dec[1, :128] == 4) and np.all(dec[1, 128:] == 8)


@pytest.mark.parametrize("group", [32, 64, 128, 256])
def test_decode_and_bf16_dequant_brute_force(group):
    n, k = 6, 512
    g = inputs.rng(31 + group)
    w = inputs.q2_0_weight(g, n, k, group)
    codes, scales = _py_unpack(w, n, k, group)
    ref = np.repeat(scales, group, axis=1) * (codes - 2)
    assert np.array_equal(oracle.q2_0_decode(w, n, k, group), ref)
    # bf16 dequant: one rounding of the exact value, rounded by torch
    ref16 = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.dequant_q2_0_to_bf16(w, n, k, group), ref16)
    # the packer agrees with the unpacker
    assert np.array_equal(_q2_weight(codes, scales, group), w)


def _tiny(seed, m=5, n=7, k=512, outliers=True):
    g = inputs.rng(seed)
    w = inputs.q2_0_weight(g, n, k)
    a = inputs.activations(g, m, k, outliers=outliers)
    q8, _ = oracle.quantize_act_q8_1(a, m, k)
    return w, a, q8


def _py_q8(q8, m, k):
    kp = oracle.q8_1_kpad(k)
    codes = q8[: m * kp].view(np.int8).reshape(m, kp)[:, :k].astype(np.int64)
    d = q8[m * kp:].view(np.float16).reshape(m, kp // 32, 2)[:, : k // 32, 0].astype(np.float64)
    return codes, d


@pytest.mark.parametrize("seed", [41, 42, 43])
def test_mmq_brute_force_and_blockdots(seed):
    m, n, k = 5, 7, 512
    w, a, q8 = _tiny(seed, m, n, k)
    codes, scales = _py_unpack(w, n, k, 128)
    qa, da = _py_q8(q8, m, k)
    A = np.repeat(da, 32, axis=1) * qa
    W = np.repeat(scales, 128, axis=1) * (codes - 2)
    ref = A @ W.T
    R = oracle.q2_0_mmq(q8, w, m, n, k)
    assert np.max(np.abs(R - ref)) <= 1e-12 * np.max(np.abs(ref))
    # integer block dots: D[i][j][b] = sum (c - 2) q over block b, exact
    D = oracle.q2_0_blockdots(q8, w, m, n, k)
    Dref = np.einsum("ibt,jbt->ijb", qa.reshape(m, k // 32, 32), (codes - 2).reshape(n, k // 32, 32))
    assert np.array_equal(D, Dref)
    # per-128-group integer sums are the sums of four block dots
    # and the scaled block dots rebuild the plain result
    rebuilt = np.einsum("ib,jb,ijb->ij", da, np.repeat(scales, 4, axis=1), D.astype(np.float64))
    assert np.max(np.abs(rebuilt - R)) <= 1e-12 * np.max(np.abs(R))


def test_mmq_closed_forms():
    m, k = 3, 256
    g = inputs.rng(44)
    a = inputs.activations(g, m, k)
    q8, _ = oracle.quantize_act_q8_1(a, m, k)
    qa, da = _py_q8(q8, m, k)
    A = np.repeat(da, 32, axis=1) * qa
    ones = np.ones((4, 2))
    # all codes 2 -> exactly zero
    w2 = _q2_weight(np.full((4, k), 2), ones, 128)
    assert not oracle.q2_0_mmq(q8, w2, m, 4, k).any()
    # codes 3, d = 1 -> every column is the row sum of the dequantized activations
    w3 = _q2_weight(np.full((4, k), 3), ones, 128)
    R3 = oracle.q2_0_mmq(q8, w3, m, 4, k)
    for j in range(4):
        assert np.allclose(R3[:, j], A.sum(1), rtol=1e-14, atol=0)
    # one-hot: code 3 at k = 77 (else 2), d = 1 -> picks column 77
    c = np.full((1, k), 2)
    c[0, 77] = 3
    R1 = oracle.q2_0_mmq(q8, _q2_weight(c, np.ones((1, 2)), 128), m, 1, k)
    assert np.array_equal(R1[:, 0], A[:, 77])


def test_mmq_integer_case():
    # a block whose amax is 127 has d = 1 and q = x; integer activations in
    # [-127, 127] with one 127 per block, weights with d = 1 -> exact integers.
    m, n, k = 2, 3, 256
    g = inputs.rng(45)
    x = g.integers(-127, 128, size=(m, k)).astype(np.float32)
    x[:, ::32] = 127
    a = inputs.f32_to_bf16_bits(x)
    q8, _ = oracle.quantize_act_q8_1(a, m, k)
    codes = g.integers(0, 4, size=(n, k))
    w = _q2_weight(codes, np.ones((n, 2)), 128)
    R = oracle.q2_0_mmq(q8, w, m, n, k)
    assert np.array_equal(R, x.astype(np.float64) @ (codes - 2).T.astype(np.float64))


def test_gemv_brute_force_and_closed_forms():
    m, n, k = 3, 9, 512
    g = inputs.rng(46)
    w = inputs.q2_0_weight(g, n, k)
    a = inputs.activations(g, m, k, outliers=True)
    codes, scales = _py_unpack(w, n, k, 128)
    X = inputs.bf16_bits_to_f32(a).astype(np.float64)
    W = np.repeat(scales, 128, axis=1) * (codes - 2)
    R = oracle.q2_0_gemv(a, w, m, n, k)
    assert np.max(np.abs(R - X @ W.T)) <= 1e-12 * np.max(np.abs(R))
    ones = np.ones((2, 4))
    assert not oracle.q2_0_gemv(a, _q2_weight(np.full((2, k), 2), ones, 128), m, 2, k).any()
    R3 = oracle.q2_0_gemv(a, _q2_weight(np.full((2, k), 3), ones, 128), m, 2, k)
    assert np.allclose(R3[:, 0], X.sum(1), rtol=1e-14, atol=0) and np.array_equal(R3[:, 0], R3[:, 1])
    xi = g.integers(-50, 50, size=(m, k)).astype(np.float32)
    Ri = oracle.q2_0_gemv(inputs.f32_to_bf16_bits(xi), _q2_weight(codes, np.ones((n, 4)), 128), m, n, k)
    assert np.array_equal(Ri, xi.astype(np.float64) @ (codes - 2).T.astype(np.float64))


def test_gemv_row_independent_of_batch():
    n, k = 6, 256
    g = inputs.rng(47)
    w = inputs.q2_0_weight(g, n, k)
    a = inputs.activations(g, 8, k)
    R8 = oracle.q2_0_gemv(a, w, 8, n, k)
    R2 = oracle.q2_0_gemv(a[:2], w, 2, n, k)
    assert np.array_equal(R8[:2], R2)


def test_dense_gemm_bf16_matches_numpy():
    m, n, k = 4, 6, 96
    g = inputs.rng(48)
    a = inputs.activations(g, m, k)
    wb = inputs.activations(g, n, k)
    ref = inputs.bf16_bits_to_f32(a).astype(np.float64) @ inputs.bf16_bits_to_f32(wb).astype(np.float64).T
    assert np.allclose(oracle.dense_gemm_bf16(a, wb, m, n, k), ref, rtol=1e-13, atol=1e-13)


def test_silu_mul():
    g = inputs.rng(49)
    gate = inputs.activations(g, 1, 4096)[0]
    up = inputs.activations(g, 1, 4096)[0]
    gate[:4] = inputs.f32_to_bf16_bits(np.array([0.0, 40.0, -40.0, 1.0], np.float32))
    up[:4] = inputs.f32_to_bf16_bits(np.array([3.0, 2.0, 2.0, 1.0], np.float32))
    out = oracle.silu_mul_bf16(gate, up)
    y = inputs.bf16_bits_to_f32(out).astype(np.float64)
    # closed forms: silu(0) = 0; silu(40) = 40 (1 - 4e-18) -> 80 after rounding;
    # silu(-40) ~ -1.7e-16 -> tiny; silu(1) = 1/(1+e^-1)
    assert y[0] == 0.0 and y[1] == 80.0 and abs(y[2]) < 1e-15
    assert y[3] == float(torch.tensor(1.0 / (1.0 + np.exp(-1.0)), dtype=torch.float64).to(torch.bfloat16))
    gv = inputs.bf16_bits_to_f32(gate).astype(np.float64)
    uv = inputs.bf16_bits_to_f32(up).astype(np.float64)
    ref = torch.nn.functional.silu(torch.from_numpy(gv)).numpy() * uv
    # within one bf16 step of libm/torch's fp64 value
    assert np.all(np.abs(y - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-30)

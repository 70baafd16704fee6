"""Pins of the oracle's Q4_K routines (decode, block dots, MMQ).

The pages fix 256 weights per block_q4_K in 144 bytes (page
layers/ops/q4k_mmq.rs, consts QK_K, Q4K_BLOCK_BYTES, fn q4k_weight_bytes); the
byte layout adopted is the public GGUF block_q4_K.  Pins: hand-packed scale
bytes whose sub-scales/mins are worked out by hand (including the j >= 4
high bits), nibble placement, brute force through an independent unpacker,
the block-dot identity, and closed forms.
"""
import numpy as np
import pytest

import inputs
import oracle
import q4k_pack

# Twelve scale bytes and their sub-scales/mins, worked by hand:
# j < 4 : sc = S[j] & 63 -> 1, 2, 3, 4 ; m = S[j+4] & 63 -> 5, 6, 7, 8
# j = 4 : sc = (0x9A & 15 = 10) | ((0xC1 >> 6 = 3) << 4) = 58 ; m = (0x9A >> 4 = 9) | ((0xC5 >> 6 = 3) << 4) = 57
# j = 5 : sc = (0xBC & 15 = 12) | ((0x82 >> 6 = 2) << 4) = 44 ; m = (11) | ((0x86 >> 6 = 2) << 4) = 43
# j = 6 : sc = (0xDE & 15 = 14) | ((0x43 >> 6 = 1) << 4) = 30 ; m = (13) | ((0x47 >> 6 = 1) << 4) = 29
# j = 7 : sc = (0xF0 & 15 = 0) | ((0x04 >> 6 = 0) << 4) = 0   ; m = (15) | ((0x08 >> 6 = 0) << 4) = 15
S_HAND = [0xC1, 0x82, 0x43, 0x04, 0xC5, 0x86, 0x47, 0x08, 0x9A, 0xBC, 0xDE, 0xF0]
SC_HAND = [1, 2, 3, 4, 58, 44, 30, 0]
M_HAND = [5, 6, 7, 8, 57, 43, 29, 15]


def _block(d, dmin, S, qs):
    b = np.zeros(144, np.uint8)
    b[0:2] = np.array([d], np.float16).view(np.uint8)
    b[2:4] = np.array([dmin], np.float16).view(np.uint8)
    b[4:16] = S
    b[16:] = qs
    return b


def test_size():
    assert oracle.q4k_bytes(17408, 5120) == 17408 * 20 * 144 == 50135040


def test_hand_scales_and_mins():
    # all codes 1: w = d*sc_j - dmin*m_j; all codes 0: w = -dmin*m_j
    one = _block(1.0, 1.0, S_HAND, np.full(128, 0x11, np.uint8))
    zero = _block(1.0, 1.0, S_HAND, np.zeros(128, np.uint8))
    d1 = oracle.q4k_decode(one, 1, 256)[0].reshape(8, 32)
    d0 = oracle.q4k_decode(zero, 1, 256)[0].reshape(8, 32)
    for j in range(8):
        assert np.all(d1[j] == SC_HAND[j] - M_HAND[j])
        assert np.all(d0[j] == -M_HAND[j])


def test_nibble_placement():
    # sc = 1, m = 0 for every sub-block: S[0..3] = 1, S[4..7] = 0, S[8..11] = 0x01.
    S = [1, 1, 1, 1, 0, 0, 0, 0, 1, 1, 1, 1]
    qs = np.zeros(128, np.uint8)
    qs[32 * 2 + 7] = 0x95  # chunk t = 2, i = 7: low nibble 5 -> weight 135, high 9 -> weight 167
    dec = oracle.q4k_decode(_block(1.0, 0.0, S, qs), 1, 256)[0]
    expect = np.zeros(256)
    expect[64 * 2 + 7] = 5
    expect[64 * 2 + 32 + 7] = 9
    assert np.array_equal(dec, expect)


_py_unpack_q4k = q4k_pack.unpack


@pytest.mark.parametrize("seed", [51, 52])
def test_brute_force_and_blockdots(seed):
    m, n, k = 4, 5, 512
    g = inputs.rng(seed)
    w = inputs.q4k_weight(g, n, k)
    a = inputs.activations(g, m, k, outliers=True)
    q8, _ = oracle.quantize_act_q8_1(a, m, k)
    codes, scale, mins = _py_unpack_q4k(w, n, k)
    W = scale * codes - mins
    assert np.array_equal(oracle.q4k_decode(w, n, k), W)
    kp = oracle.q8_1_kpad(k)
    qa = q8[: m * kp].view(np.int8).reshape(m, kp)[:, :k].astype(np.int64)
    da = q8[m * kp:].view(np.float16).reshape(m, kp // 32, 2)[:, : k // 32, 0].astype(np.float64)
    A = np.repeat(da, 32, axis=1) * qa
    R = oracle.q4k_mmq(q8, w, m, n, k)
    ref = A @ W.T
    assert np.max(np.abs(R - ref)) <= 1e-12 * np.max(np.abs(ref))
    D = oracle.q4k_blockdots(q8, w, m, n, k)
    Dref = np.einsum("ibt,jbt->ijb", qa.reshape(m, k // 32, 32), codes.reshape(n, k // 32, 32))
    assert np.array_equal(D, Dref)
    # R = sum_j [ d*sc_j * d_a * D_j - dmin*m_j * d_a * Q_j ]
    Q = qa.reshape(m, k // 32, 32).sum(-1).astype(np.float64)
    sc_b = scale[:, ::32]
    mn_b = mins[:, ::32]
    rebuilt = np.einsum("ib,jb,ijb->ij", da, sc_b, D.astype(np.float64)) - np.einsum("ib,jb,ib->ij", da, mn_b, Q)
    assert np.max(np.abs(rebuilt - R)) <= 1e-12 * np.max(np.abs(R))


def test_closed_forms():
    m, k = 3, 256
    g = inputs.rng(53)
    a = inputs.activations(g, m, k)
    q8, _ = oracle.quantize_act_q8_1(a, m, k)
    A = oracle.dequant_q8_1(q8, m, k)[:, :k]
    # dmin = 0, sc = 1, d = 1 -> plain uint4 GEMM
    S1 = [1, 1, 1, 1, 0, 0, 0, 0, 1, 1, 1, 1]
    qs = g.integers(0, 256, 128, dtype=np.uint8)
    w = _block(1.0, 0.0, S1, qs)
    codes = np.stack([qs.reshape(4, 32) & 15, qs.reshape(4, 32) >> 4], 1).reshape(256).astype(np.float64)
    assert np.allclose(oracle.q4k_mmq(q8, w, m, 1, k)[:, 0], A @ codes, rtol=1e-14, atol=0)
    # sc = 0, m = 1, dmin = 1 -> R = -sum_k deq(a)
    Sm = [0, 0, 0, 0, 1, 1, 1, 1, 0x10, 0x10, 0x10, 0x10]
    w = _block(1.0, 1.0, Sm, qs)
    assert np.allclose(oracle.q4k_mmq(q8, w, m, 1, k)[:, 0], -A.sum(1), rtol=1e-14, atol=0)

"""Pins of the oracle's q8_1 activation quantizer.

The pages name the encoding (blocks of 32 int8 values with a scale d and a
sum s, rows padded to 256: page layers/ops/q4k_mmq.rs, fn quantize_act_q8_1)
but print no rule and no worked example.  The rule adopted is: d =
fp16(amax/127), q = clamp(roundf(x/d), +-127) with the stored d, s =
fp16(d * sum q).  What pins the oracle to it, independently of its code:
  * hand-worked blocks (values derived below by hand),
  * brute force: every code is a nearest integer multiple of d,
  * the invariants named for the format (s equals the code sum times d;
    round trip within half a step; |q| = 127 at the block maximum),
  * a ties block that separates ties-away from ties-to-even.
"""
import numpy as np
import pytest

import inputs
import oracle


def _unpack(q8, m, k):
    kp = oracle.q8_1_kpad(k)
    codes = q8[: m * kp].view(np.int8).reshape(m, kp)
    ds = q8[m * kp:].view(np.uint16).reshape(m, kp // 32, 2)
    return codes, ds[..., 0], ds[..., 1]


def _bf16(x):
    return inputs.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_sizes_and_padding():
    assert oracle.q8_1_kpad(512) == 512
    assert oracle.q8_1_kpad(1) == 256
    assert oracle.q8_1_kpad(257) == 512
    # codes plane + one 4-byte (d, s) pair per 32 values = 1.125 bytes per value
    assert oracle.q8_1_bytes(3, 300) == 3 * 512 + 3 * 16 * 4
    a = _bf16(np.full((2, 40), 3.0))
    q8, flagged = oracle.quantize_act_q8_1(a, 2, 40)
    codes, d, s = _unpack(q8, 2, 40)
    assert flagged == 0
    assert np.all(codes[:, :40] == 127) and np.all(codes[:, 40:] == 0)
    assert np.all(d[:, 2:] == 0) and np.all(s[:, 2:] == 0)


def test_worked_example_ramp():
    # x_i = i, i = 0..31 (exact in bf16).  amax = 31; 31/127 = 0.2440944...;
    # binary16 spacing there is 2^-12, 0.2440944 * 4096 = 999.81 -> 1000,
    # so d = 1000/4096 = 0.244140625 = 1.953125 * 2^-3 -> bits 0x33D0.
    # q_i = roundf(i / 0.244140625) = roundf(4.096 i).
    # sum q = 2031; s = fp16(0.244140625 * 2031 = 495.849609375); spacing at
    # 495 is 2^-2, 495.8496 / 0.25 = 1983.4 -> 1983 * 0.25 = 495.75 -> 0x5FBF.
    x = np.arange(32, dtype=np.float32)[None, :]
    q8, _ = oracle.quantize_act_q8_1(_bf16(x), 1, 32)
    codes, d, s = _unpack(q8, 1, 32)
    expect = [0, 4, 8, 12, 16, 20, 25, 29, 33, 37, 41, 45, 49, 53, 57, 61, 66, 70, 74, 78,
              82, 86, 90, 94, 98, 102, 106, 111, 115, 119, 123, 127]
    assert codes[0, :32].tolist() == expect
    assert sum(expect) == 2031
    assert d[0, 0] == 0x33D0 and s[0, 0] == 0x5FBF


def test_worked_example_alternating_with_outlier():
    # x_i = (-1)^i (i+1)/8, with x_5 (= -0.75) times 20 = -15.  All exact in bf16.
    # amax = 15; 15/127 = 0.1181102...; spacing 2^-14 there, 0.1181102 * 16384 =
    # 1935.1 -> 1935/16384 = 0.11810302734375 = bits 0x2F8F.
    # q_i = roundf(x_i / d) = roundf(x_i * 8.4672...).  Hand values below; q_5 = -127.
    # sum q = -138; s = fp16(d * -138 = -16.29821777...) spacing 2^-6 -> -1043.08/64
    # -> -1043 * 2^-6 = -16.296875 = bits 0xCC13.
    x = np.array([(-1) ** i * (i + 1) / 8 for i in range(32)], dtype=np.float32)
    x[5] *= 20
    q8, _ = oracle.quantize_act_q8_1(_bf16(x[None, :]), 1, 32)
    codes, d, s = _unpack(q8, 1, 32)
    expect = [1, -2, 3, -4, 5, -127, 7, -8, 10, -11, 12, -13, 14, -15, 16, -17, 18, -19, 20,
              -21, 22, -23, 24, -25, 26, -28, 29, -30, 31, -32, 33, -34]
    assert codes[0, :32].tolist() == expect
    assert sum(expect) == -138
    assert d[0, 0] == 0x2F8F and s[0, 0] == 0xCC13


def test_ties_round_away_from_zero():
    # amax = 127 gives d = 127/127 = 1 exactly, so q = roundf(x): halves go away
    # from zero (2.5 -> 3, -0.5 -> -1); ties-to-even would give 2 and 0.
    vals = [127.0, 2.5, -2.5, 0.5, -0.5, 126.5, -1.5, 3.5] + [0.0] * 24
    q8, _ = oracle.quantize_act_q8_1(_bf16(np.array(vals)[None, :]), 1, 32)
    codes, d, s = _unpack(q8, 1, 32)
    assert d[0, 0] == 0x3C00
    assert codes[0, :8].tolist() == [127, 3, -3, 1, -1, 127, -2, 4]


def test_zero_block():
    q8, _ = oracle.quantize_act_q8_1(_bf16(np.zeros((1, 64))), 1, 64)
    codes, d, s = _unpack(q8, 1, 64)
    assert not codes.any() and not d.any() and not s.any()


@pytest.mark.parametrize("seed,outliers", [(21, False), (22, True), (23, True)])
def test_invariants_and_brute_force(seed, outliers):
    m, k = 24, 1024
    g = inputs.rng(seed)
    a = inputs.activations(g, m, k, outliers=outliers)
    # add some tiny and zero rows to reach subnormal and zero scales
    a[0] = inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(a[0]) * np.float32(1e-6))
    a[1, :64] = 0
    q8, flagged = oracle.quantize_act_q8_1(a, m, k)
    assert flagged == 0
    codes, dbits, sbits = _unpack(q8, m, k)
    x = inputs.bf16_bits_to_f32(a).astype(np.float64).reshape(m, k // 32, 32)
    q = codes.astype(np.int64).reshape(m, k // 32, 32)
    d = dbits.view(np.float16).astype(np.float64)
    s = sbits.view(np.float16)
    # s is the binary16 rounding of d times the code sum (numpy's own rounding)
    s_ref = (d.astype(np.float32) * q.sum(-1).astype(np.float32)).astype(np.float16)
    assert np.array_equal(s.view(np.uint16), s_ref.view(np.uint16))
    # d is the binary16 rounding of amax/127 taken in binary32
    amax = np.abs(x).max(-1).astype(np.float32)
    assert np.array_equal(dbits, (amax / np.float32(127)).astype(np.float16).view(np.uint16))
    # brute force nearest integer over [-127, 127], and round trip within half a step
    cand = np.arange(-127, 128, dtype=np.float64)
    dd = d[..., None]
    nz = d > 0
    err = np.abs(x - dd * q)
    best = np.abs(x[..., None] - dd[..., None] * cand).min(-1)
    slack = dd * 2.0 ** -16
    assert np.all((err <= best + slack)[nz])
    unclamped = np.abs(q) < 127
    assert np.all(((err <= dd * (0.5 + 2.0 ** -16)) | ~unclamped)[nz])
    # |q| = 127 at the block maximum for normal-range scales
    normal = d >= 2.0 ** -14
    at_max = np.take_along_axis(np.abs(q), np.abs(x).argmax(-1)[..., None], -1)[..., 0]
    assert np.all((at_max == 127)[normal])
    # zero scale -> zero codes and zero sum
    assert not q[~nz].any() and not s[~nz].view(np.uint16).any()


def test_out_of_range_is_flagged():
    a = _bf16(np.array([[3000.0] + [0.0] * 31]))
    _, flagged = oracle.quantize_act_q8_1(a, 1, 32)
    assert flagged == 1

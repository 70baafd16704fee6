"""Pins of the oracle's Q4_K decode GEMV and Q4_K weight quantizer.

GEMV (the product of bf16 activations and the dequantized Q4_K weight, page
layers/ops/q4k_mmq.rs, fn q4k_mmq_gemm, taken without the q8_1 step): brute
force against a numpy fp64 matmul of the independently unpacked weight, and
the one-hot closed form.

Quantizer (page layers/ops/q4k_mmq.rs, fn quantize_weight_q4k; the page gives
no rule, the oracle states the affine min/max reading it adopts):
  * exact recovery: blocks built from chosen (d, dmin, sc_j, m_j, codes),
    whose sub-block extremes and scale maxima are exact in bf16/fp16, must
    come back byte for byte as packed by the test's own packer;
  * a bound derived from the reading: with S_j and M_j the unrounded step and
    offset, |sc_j d - S_j| <= d/2 and |m_j dmin - M_j| <= dmin/2, so a value
    inside the code range is off by at most half a stored step, a value
    clamped at 15 by at most 7.5 d + dmin/2, one clamped at 0 by at most
    dmin/2:  |x - deq(x)| <= max(d sc_j / 2, 7.5 d + dmin / 2);
  * the zero block, a constant block, and the supported-range flag.
"""
import numpy as np
import pytest

import inputs
import oracle
import q4k_pack


# --- GEMV ------------------------------------------------------------------

@pytest.mark.parametrize("m,n,k,seed", [(1, 7, 512, 61), (3, 5, 768, 62), (8, 4, 256, 63)])
def test_gemv_brute_force(m, n, k, seed):
    g = inputs.rng(seed)
    w = inputs.q4k_weight(g, n, k)
    a = inputs.activations(g, m, k, outliers=True)
    A = inputs.bf16_bits_to_f32(a).astype(np.float64)
    ref = A @ q4k_pack.dequant(w, n, k).T
    R = oracle.q4k_gemv(a, w, m, n, k)
    assert np.max(np.abs(R - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_gemv_one_hot_column():
    n, k = 6, 512
    g = inputs.rng(64)
    w = inputs.q4k_weight(g, n, k)
    W = q4k_pack.dequant(w, n, k)
    for col in (0, 37, 255, 300, 511):
        a = np.zeros((1, k), np.uint16)
        a[0, col] = 0x3F80  # bf16 1.0
        assert np.array_equal(oracle.q4k_gemv(a, w, 1, n, k)[0], W[:, col])


# --- quantizer -------------------------------------------------------------

def _bf16(x):
    return inputs.f32_to_bf16_bits(np.asarray(x, np.float32))


def _sig_bits_ok(v):
    """|v| has at most 8 significant bits (exact in bf16)."""
    v = abs(int(v))
    while v and v % 2 == 0:
        v //= 2
    return v <= 255


def _exact_block(g):
    """(bf16 values [256], expected bytes [144]).  d = 2^-10, dmin = 2^-11,
    x = d sc q - dmin m = 2^-11 (2 sc q - m).  Every sub-block holds q = 0
    and q = 15, so lo = -dmin m and hi = 2^-11 (30 sc - m) are its extremes;
    (sc, m) are chosen so that hi is exact in bf16, sub-block 0 has sc = 63
    and sub-block 1 has m = 63, so max S / 63 = d and max M / 63 = dmin
    exactly.  sc >= 8 keeps the bf16 rounding of the other values
    (<= 2^-9 |x| <= 1.9 d) under half a step."""
    d, dmin = 2.0 ** -10, 2.0 ** -11
    sc = np.zeros(8, np.int64)
    mn = np.zeros(8, np.int64)
    sc[0], mn[0] = 63, int(g.choice([2, 10]))
    sc[1], mn[1] = int(g.choice([8, 9, 10])), 63
    for j in range(2, 8):
        while True:
            s, m_ = int(g.integers(8, 64)), int(g.integers(0, 64))
            if _sig_bits_ok(30 * s - m_):
                sc[j], mn[j] = s, m_
                break
    codes = g.integers(0, 16, size=(8, 32))
    for j in range(8):
        p = g.permutation(32)[:2]
        codes[j, p[0]], codes[j, p[1]] = 0, 15
    x = (d * sc[:, None] * codes - dmin * mn[:, None]).reshape(256)
    return _bf16(x), q4k_pack.pack_block(d, dmin, sc, mn, codes.reshape(256))


@pytest.mark.parametrize("seed", [71, 72, 73])
def test_quantize_exact_recovery(seed):
    g = inputs.rng(seed)
    rows = [_exact_block(g) for _ in range(6)]
    xs = np.concatenate([r[0] for r in rows]).reshape(2, 768)  # 2 rows of 3 super-blocks
    expect = np.concatenate([r[1] for r in rows])
    got, flagged = oracle.quantize_weight_q4k(xs, 2, 768)
    assert flagged == 0
    assert np.array_equal(got, expect)


def _check_bound(x_bits, n, k):
    q, flagged = oracle.quantize_weight_q4k(x_bits, n, k)
    assert flagged == 0
    x = inputs.bf16_bits_to_f32(x_bits.reshape(n, k)).astype(np.float64)
    deq = q4k_pack.dequant(q, n, k)
    d, dmin, sc, mn = q4k_pack.fields(q, n, k)
    step = np.repeat(d[..., None] * sc, 32, -1).reshape(n, k)
    clampb = np.repeat(np.broadcast_to((7.5 * d + 0.5 * dmin)[..., None], sc.shape), 32, -1).reshape(n, k)
    bound = np.maximum(0.5 * step, clampb)
    slack = 1e-6 * np.abs(x) + 1e-30
    assert np.all(np.abs(x - deq) <= bound * (1 + 1e-6) + slack)
    # fields are in range, d and dmin are the fp16 roundings of the scale maxima / 63
    assert sc.max() <= 63 and mn.max() <= 63
    return q, x, deq


@pytest.mark.parametrize("seed,scale", [(81, 0.02), (82, 1.0), (83, 2e-4)])
def test_quantize_error_bound(seed, scale):
    n, k = 5, 1024
    g = inputs.rng(seed)
    x = g.standard_normal((n, k)).astype(np.float32) * scale
    x[0, 0:32] = np.abs(x[0, 0:32]) + scale        # all positive sub-block
    x[0, 32:64] = -np.abs(x[0, 32:64]) - scale     # all negative
    x[1, 0:32] = 0.5 * scale                       # constant
    x[1, 64:96] = 0.0                              # zero sub-block
    x[2, 300] = 40 * scale                         # outlier
    x[3, 256:512] = 0.0                            # zero super-block
    _, xf, deq = _check_bound(_bf16(x), n, k)
    # the fit is useful: error well under the data's spread
    assert np.sqrt(np.mean((xf - deq) ** 2)) <= 0.2 * np.sqrt(np.mean(xf ** 2))


def test_quantize_zero_and_constant():
    z, f = oracle.quantize_weight_q4k(np.zeros(256, np.uint16), 1, 256)
    assert f == 0 and not z.any()
    negz, f = oracle.quantize_weight_q4k(np.full(256, 0x8000, np.uint16), 1, 256)  # -0.0
    assert f == 0 and not negz.any()
    c = 0.75
    q, f = oracle.quantize_weight_q4k(_bf16(np.full(256, c)), 1, 256)
    d, dmin, sc, mn = q4k_pack.fields(q, 1, 256)
    codes, _, _ = q4k_pack.unpack(q, 1, 256)
    # lo = 0 (no offset), one step of c/15 per sub-block; sc = 63, top code
    assert dmin[0, 0] == 0 and np.all(mn == 0) and np.all(sc == 63) and np.all(codes == 15)
    assert d[0, 0] == np.float64(np.float16(np.float32(c) / np.float32(15) / np.float32(63)))
    assert np.max(np.abs(q4k_pack.dequant(q, 1, 256) - c)) <= 7.5 * d[0, 0]


def test_quantize_range_flag():
    x = np.zeros((2, 512), np.float32)
    x[0, 5] = np.inf
    x[1, 300] = 3.0e38                              # d overflows binary16
    _, f = oracle.quantize_weight_q4k(_bf16(x), 2, 512)
    assert f == 2


# --- the quantizer's rounding of exact ties ----------------------------------

def _round_half_away(q):
    """Nearest integer to the Fraction q, halves away from zero."""
    from fractions import Fraction
    f = q.numerator // q.denominator
    r = q - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and q > 0):
        return f + 1
    if r == Fraction(1, 2) and q < 0:
        return f
    return f if r < Fraction(1, 2) else f + 1


def _round_half_even(q):
    from fractions import Fraction
    f = q.numerator // q.denominator
    r = q - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        return f + 1
    return f


def _tie_block():
    """A super-block whose sub-scale, sub-min and code quotients land exactly
    on halves, with every value and intermediate exact (values in units of
    u = 2^-13, all with <= 8 significant bits, so exact in bf16; d and dmin
    come out as u exactly).  Returns (bf16 bits [256], the sub-blocks' values
    as Fractions in units of u, the number of exact ties)."""
    from fractions import Fraction as F
    h = F(1, 2)
    # per sub-block: the values in units of u (the extremes first)
    sub = [
        [F(-49), F(896), F(0), F(448)],          # S = 63u, M = 49u: sets d = u
        [F(-63), F(57), F(-43), F(-27), F(-11), F(-59), F(53)],  # M = 63u sets dmin = u; sc = 8,
                                                 # codes (x + 63) / 8 = 2.5, 4.5, 6.5, 0.5, 14.5
        [F(0), F(255) * h, F(45) * h, F(9)],     # S = 8.5u -> sc = 9 (tie); codes 2.5 and 1
        [F(-21) * h, F(129) * h, F(0)],          # M = 10.5u -> m = 11 (tie); S = 5u
        [F(-105) * h, F(255), F(0)],             # S = 20.5u -> sc = 21, M = 52.5u -> m = 53 (both ties)
        [F(0), F(60), F(30)],                    # S = 4u, codes 15 and 7.5 -> 8 (tie)
        [F(-5), F(25), F(1)],                    # S = 2u, M = 5u: codes (1 + 5) / 2 = 3
        [F(0)],                                  # a zero sub-block
    ]
    vals = []
    for j, v in enumerate(sub):
        vals.append((v + [v[-1]] * 32)[:32])
    x = np.array([float(v) * 2.0 ** -13 for blk in vals for v in blk], np.float64)
    bits = inputs.f32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(inputs.bf16_bits_to_f32(bits).astype(np.float64), x)  # exact in bf16
    return bits, vals


def _expected_tie_bytes(vals, rnd):
    """The quantizer's rule in exact rationals (units of u) with rounding rnd."""
    from fractions import Fraction as F
    lo = [min(F(0), min(v)) for v in vals]
    hi = [max(l, max(v)) for l, v in zip(lo, vals)]
    S = [(h - l) / 15 for h, l in zip(hi, lo)]
    M = [-l for l in lo]
    d, dmin = max(S) / 63, max(M) / 63
    assert d == 1 and dmin == 1  # both exactly u, so fp16(u) = u
    sc = [min(63, rnd(s / d)) for s in S]
    mn = [min(63, rnd(m_ / dmin)) for m_ in M]
    codes, ties = [], 0
    for j, v in enumerate(vals):
        for x in v:
            step = d * sc[j]
            q = 0 if step == 0 else max(0, min(15, rnd((x + dmin * mn[j]) / step)))
            if step != 0 and ((x + dmin * mn[j]) / step).denominator == 2:
                ties += 1
            codes.append(q)
    ties += sum(1 for s in S if (s / d).denominator == 2) + sum(1 for m_ in M if (m_ / dmin).denominator == 2)
    return q4k_pack.pack_block(2.0 ** -13, 2.0 ** -13, sc, mn, np.array(codes)), ties


def test_quantize_ties_away_from_zero():
    # exact halves in S_j/d, M_j/dmin and the code quotients round away from
    # zero (roundf), as the quantizer's reading fixes; the same block under
    # ties-to-even gives other bytes, so the pin tells the two rules apart
    bits, vals = _tie_block()
    expect, ties = _expected_tie_bytes(vals, _round_half_away)
    other, _ = _expected_tie_bytes(vals, _round_half_even)
    assert ties >= 40
    assert not np.array_equal(expect, other)
    got, flagged = oracle.quantize_weight_q4k(bits, 1, 256)
    assert flagged == 0
    assert np.array_equal(got, expect)
    # the sub-scale and sub-min ties themselves: sc_2 = 9 (8.5), m_3 = 11 (10.5),
    # sc_4 = 21 (20.5), m_4 = 53 (52.5; a j >= 4 sub-block, so its high bits too)
    _, _, sc, mn = q4k_pack.fields(got, 1, 256)
    assert sc[0, 0, 2] == 9 and mn[0, 0, 3] == 11 and sc[0, 0, 4] == 21 and mn[0, 0, 4] == 53

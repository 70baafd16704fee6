"""Pins of the oracle's scalar conversions against independent library
routines (numpy's binary16, torch's bfloat16) and exact rational arithmetic."""
from fractions import Fraction

import numpy as np
import torch

import oracle


def test_f16_to_f32_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_to_f32(int(b)) for b in bits], dtype=np.float32)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.all(np.isnan(got[np.isnan(ref)]))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def _f16_cases():
    g = np.random.Generator(np.random.PCG64(11))
    xs = [g.standard_normal(4000).astype(np.float32) * s for s in (1e-6, 1e-4, 0.02, 1.0, 300.0, 3e4)]
    xs = np.concatenate(xs)
    special = []
    for e in range(-26, 16):
        base = np.float32(2.0 ** e)
        # exact ties between binary16 neighbours and their neighbours
        ulp = 2.0 ** (max(e, -14) - 10)
        for j in range(0, 6):
            special += [base + np.float32((j + 0.5) * ulp), base + np.float32(j * ulp)]
    special += [65504.0, 65519.996, 65520.0, 70000.0, 2.0 ** -25, 2.0 ** -25 * 1.0000001,
                2.0 ** -24 * 1.5, 2.0 ** -24 * 2.5, 0.0, 1e-30, 1e-45]
    sp = np.array(special, dtype=np.float32)
    return np.concatenate([xs, sp, -sp])


def test_f32_to_f16_matches_numpy_rne():
    xs = _f16_cases()
    ref = xs.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16(float(x)) for x in xs], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(xs[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


def test_bf16_to_f64_all_patterns():
    bits = np.arange(65536, dtype=np.uint32)
    ref = (bits << 16).view(np.float32).astype(np.float64)
    got = np.array([oracle.bf16_to_f64(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])


def test_f64_to_bf16_on_floats_matches_torch():
    # For binary32 inputs one rounding to bf16 is what torch does.
    g = np.random.Generator(np.random.PCG64(12))
    xs = np.concatenate([g.standard_normal(20000).astype(np.float32) * s for s in (1e-38, 1e-3, 1.0, 1e30)])
    ref = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f64_to_bf16(float(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, ref)


def _bf16_exact_rne(x: float) -> int:
    """Brute force: nearest of the two bf16 neighbours of x by exact rationals,
    ties to the even significand."""
    fx = Fraction(x)
    f32 = np.float32(x)
    cand = set()
    b = int(np.array([f32]).view(np.uint32)[0] >> 16)
    for d in (-1, 0, 1, 2):
        bb = (b + d) & 0xFFFF
        cand.add(bb)
    best = None
    for bb in cand:
        v = np.array([bb << 16], dtype=np.uint32).view(np.float32)[0]
        if not np.isfinite(v):
            continue
        err = abs(Fraction(float(v)) - fx)
        key = (err, bb & 1)
        if best is None or key < best[0]:
            best = (key, bb)
    return best[1]


def test_f64_to_bf16_single_rounding_brute_force():
    # doubles near bf16 ties, where rounding through binary32 would round twice
    g = np.random.Generator(np.random.PCG64(13))
    xs = []
    for _ in range(3000):
        e = int(g.integers(-20, 20))
        sig = int(g.integers(128, 256))
        tie = (sig + 0.5) * 2.0 ** (e - 7)
        xs += [tie, tie * (1 + 2.0 ** -40), tie * (1 - 2.0 ** -40), -tie * (1 + 2.0 ** -30)]
    for x in xs:
        assert oracle.f64_to_bf16(x) == _bf16_exact_rne(x), x

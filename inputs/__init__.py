"""Seeded synthetic inputs shared by the tests and the benchmark.

This module holds none of the method's arithmetic: it draws random numbers
and lays them into the byte containers of the formats (codes planes, scale
planes, super-block fields).  It imports neither the oracle nor the HIP
binding, and both sides receive the same arrays from it.

Recipe (numpy PCG64, one Generator per seed, draws in the order listed):
  Q2_0 weight [n, k], group 128:
    1. codes plane: n*k/4 uniform random bytes.  A byte holds four 2-bit
       codes, so uniform bytes are exactly four independent codes uniform
       in {0, 1, 2, 3}.
    2. scales: fp16(|N(0, 0.02)|), one per (row, group), row-major [n][k/128].
  Q4_K weight [n, k], 256-weight super-blocks of 144 bytes:
    1. d   = fp16(|N(0, 0.02)| / 64) per super-block,
    2. dmin = fp16(|N(0, 0.02)| / 64) per super-block,
    3. the 12 packed scale/min bytes uniform: every 6-bit sub-scale and
       sub-min is then an independent uniform draw from 0..63,
    4. the 128 code bytes uniform: independent uniform 4-bit codes.
  Activations [m, k]:
    1. standard normal (float32),
    2. where outliers are asked for, round(0.01 k) distinct columns chosen
       uniformly, multiplied by 20 in every row,
    3. rounded to bf16, nearest-even.
Multi-weight workloads draw their weights in the order gate, up, down, then
the activations.
"""
from __future__ import annotations

import numpy as np

GROUP = 128


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def q2_0_weight(g: np.random.Generator, n: int, k: int, group: int = GROUP) -> np.ndarray:
    """Packed Q2_0 weight bytes: codes plane then fp16 scale plane."""
    assert k % group == 0 and group % 4 == 0
    codes = g.integers(0, 256, size=n * k // 4, dtype=np.uint8)
    scales = np.abs(g.normal(0.0, 0.02, size=(n, k // group))).astype(np.float16)
    return np.concatenate([codes, scales.reshape(-1).view(np.uint8)])


def q4k_weight(g: np.random.Generator, n: int, k: int) -> np.ndarray:
    """Packed Q4_K weight bytes, [n][k/256] super-blocks of 144 bytes."""
    assert k % 256 == 0
    nsb = n * (k // 256)
    d = (np.abs(g.normal(0.0, 0.02, size=nsb)) / 64.0).astype(np.float16)
    dmin = (np.abs(g.normal(0.0, 0.02, size=nsb)) / 64.0).astype(np.float16)
    sc = g.integers(0, 256, size=(nsb, 12), dtype=np.uint8)
    qs = g.integers(0, 256, size=(nsb, 128), dtype=np.uint8)
    blk = np.empty((nsb, 144), dtype=np.uint8)
    blk[:, 0:2] = d.view(np.uint8).reshape(nsb, 2)
    blk[:, 2:4] = dmin.view(np.uint8).reshape(nsb, 2)
    blk[:, 4:16] = sc
    blk[:, 16:144] = qs
    return blk.reshape(-1)


def bf16_weight(g: np.random.Generator, n: int, k: int, scale: float = 0.02) -> np.ndarray:
    """bf16 bit patterns [n][k] of N(0, scale^2) weights (input of the Q4_K
    weight quantizer)."""
    return f32_to_bf16_bits(g.standard_normal(size=(n, k), dtype=np.float32) * np.float32(scale))


def activations(g: np.random.Generator, m: int, k: int, outliers: bool = False) -> np.ndarray:
    """bf16 bit patterns [m][k]: N(0,1), optionally 1% of columns times 20."""
    x = g.standard_normal(size=(m, k), dtype=np.float32)
    if outliers:
        cols = g.choice(k, size=int(round(0.01 * k)), replace=False)
        x[:, cols] *= 20.0
    return f32_to_bf16_bits(x)


# --- the five workloads -----------------------------------------------------

def tiny(seed: int = 0):
    """m=4, n=256, k=512 Q2_0; N(0,1) activations."""
    g = rng(seed)
    w = q2_0_weight(g, 256, 512)
    a = activations(g, 4, 512)
    return dict(m=4, n=256, k=512, w=w, act=a)


def decode_gemv(seed: int = 2):
    """m=1 Q2_0 in_proj_qkvz: n=12288 (2*16*128 key + 2*32*128 value/z), k=2048,
    activations with 1% outlier channels (x20)."""
    g = rng(seed)
    n, k = 12288, 2048
    w = q2_0_weight(g, n, k)
    a = activations(g, 1, k, outliers=True)
    return dict(m=1, n=n, k=k, w=w, act=a)


HIDDEN, INTER = 5120, 17408


def verify_ffn(seed: int = 3, rows: int = 8):
    """Dense SiLU FFN, Q2_0 gate/up [17408, 5120] and down [5120, 17408];
    activations [rows][5120] N(0,1); a run with m rows uses the first m."""
    g = rng(seed)
    wg = q2_0_weight(g, INTER, HIDDEN)
    wu = q2_0_weight(g, INTER, HIDDEN)
    wd = q2_0_weight(g, HIDDEN, INTER)
    a = activations(g, rows, HIDDEN)
    return dict(hidden=HIDDEN, inter=INTER, wg=wg, wu=wu, wd=wd, act=a)


def prefill_qkvz(seed: int = 4, rows: int = 2048):
    """Q2_0 qkvz n=12288, k=2048; activations [rows][2048] with 1% outlier
    channels; m=512 uses the first 512 rows."""
    g = rng(seed)
    n, k = 12288, 2048
    w = q2_0_weight(g, n, k)
    a = activations(g, rows, k, outliers=True)
    return dict(n=n, k=k, w=w, act=a)


def q4k_decode(seed: int = 6):
    """Q4_K decode (m=1) on the FFN shapes: gate/up [17408, 5120] and down
    [5120, 17408] weights, N(0,1) activations with 1% outlier channels; and a
    bf16 N(0, 0.02^2) [17408, 5120] weight for the Q4_K weight quantizer."""
    g = rng(seed)
    return dict(hidden=HIDDEN, inter=INTER,
                w_gate=q4k_weight(g, INTER, HIDDEN), a_gate=activations(g, 1, HIDDEN, outliers=True),
                w_down=q4k_weight(g, HIDDEN, INTER), a_down=activations(g, 1, INTER, outliers=True),
                w_bf16=bf16_weight(g, INTER, HIDDEN))


def prefill_ffn(seed: int = 5, rows: int = 4096, formats=("q2_0", "q4k")):
    """m=4096 FFN prefill: gate/up [17408, 5120], down [5120, 17408] in Q2_0
    and in Q4_K; N(0,1) activations [rows][5120]."""
    g = rng(seed)
    out = dict(hidden=HIDDEN, inter=INTER)
    if "q2_0" in formats:
        out["q2"] = dict(wg=q2_0_weight(g, INTER, HIDDEN), wu=q2_0_weight(g, INTER, HIDDEN),
                         wd=q2_0_weight(g, HIDDEN, INTER))
    if "q4k" in formats:
        out["q4k"] = dict(wg=q4k_weight(g, INTER, HIDDEN), wu=q4k_weight(g, INTER, HIDDEN),
                          wd=q4k_weight(g, HIDDEN, INTER))
    out["act"] = activations(g, rows, HIDDEN)
    return out

"""Independent numpy pack/unpack of the adopted block_q4_K byte layout, for
tests only (written apart from the oracle's C and the HIP kernels).

Layout (256 weights in 144 bytes): fp16 d, fp16 dmin, twelve bytes S of
6-bit sub-scales sc_j and sub-mins m_j (j < 4: sc = S[j] & 63,
m = S[j+4] & 63; j >= 4: sc = (S[j+4] & 15) | (S[j-4] >> 6) << 4,
m = (S[j+4] >> 4) | (S[j] >> 6) << 4), then 128 code bytes: byte
16 + 32t + i holds weight 64t + i in its low nibble and 64t + 32 + i in its
high nibble.  Weight value: d * sc_j * q - dmin * m_j.
"""
import numpy as np


def unpack(w, n, k):
    """codes [n][k], per-weight scale d*sc and min dmin*m (fp64)."""
    nsb = k // 256
    blk = np.asarray(w, np.uint8).reshape(n, nsb, 144)
    d = blk[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    dmin = blk[..., 2:4].copy().view(np.float16)[..., 0].astype(np.float64)
    S = blk[..., 4:16].astype(np.int64)
    sc = np.zeros((n, nsb, 8), np.int64)
    mn = np.zeros((n, nsb, 8), np.int64)
    sc[..., :4] = S[..., 0:4] & 63
    mn[..., :4] = S[..., 4:8] & 63
    sc[..., 4:] = (S[..., 8:12] & 15) | ((S[..., 0:4] >> 6) << 4)
    mn[..., 4:] = (S[..., 8:12] >> 4) | ((S[..., 4:8] >> 6) << 4)
    qs = blk[..., 16:].reshape(n, nsb, 4, 32).astype(np.int64)
    codes = np.stack([qs & 15, qs >> 4], axis=3).reshape(n, nsb, 256)  # chunk t: low then high
    scale = np.repeat(d[..., None] * sc, 32, axis=-1)
    mins = np.repeat(dmin[..., None] * mn, 32, axis=-1)
    return codes.reshape(n, k), scale.reshape(n, k), mins.reshape(n, k)


def dequant(w, n, k):
    codes, scale, mins = unpack(w, n, k)
    return scale * codes - mins


def fields(w, n, k):
    """(d, dmin) as fp64 [n][nsb] and (sc, m) as int [n][nsb][8]."""
    nsb = k // 256
    codes, scale, mins = unpack(w, n, k)
    blk = np.asarray(w, np.uint8).reshape(n, nsb, 144)
    d = blk[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    dmin = blk[..., 2:4].copy().view(np.float16)[..., 0].astype(np.float64)
    S = blk[..., 4:16].astype(np.int64)
    sc = np.concatenate([S[..., 0:4] & 63, (S[..., 8:12] & 15) | ((S[..., 0:4] >> 6) << 4)], -1)
    mn = np.concatenate([S[..., 4:8] & 63, (S[..., 8:12] >> 4) | ((S[..., 4:8] >> 6) << 4)], -1)
    return d, dmin, sc, mn


def pack_block(d, dmin, sc, mn, codes):
    """One 144-byte block from fp16 d/dmin, sc[8], m[8] (0..63), codes[256] (0..15)."""
    sc = np.asarray(sc, np.int64)
    mn = np.asarray(mn, np.int64)
    codes = np.asarray(codes, np.int64).reshape(4, 2, 32)  # chunk, (low, high), i
    assert sc.min() >= 0 and sc.max() < 64 and mn.min() >= 0 and mn.max() < 64
    assert codes.min() >= 0 and codes.max() < 16
    b = np.zeros(144, np.uint8)
    b[0:2] = np.array([d], np.float16).view(np.uint8)
    b[2:4] = np.array([dmin], np.float16).view(np.uint8)
    S = np.zeros(12, np.int64)
    S[0:4] = sc[0:4] | ((sc[4:8] >> 4) << 6)
    S[4:8] = mn[0:4] | ((mn[4:8] >> 4) << 6)
    S[8:12] = (sc[4:8] & 15) | ((mn[4:8] & 15) << 4)
    b[4:16] = S.astype(np.uint8)
    b[16:] = (codes[:, 0, :] | (codes[:, 1, :] << 4)).reshape(128).astype(np.uint8)
    return b

"""GPU parity: the BF16 dequant fallback (dequant bit-exact; dense GEMM and
the prefill dispatcher's fallback branch within relative Frobenius 2e-2), the
dispatcher's MMQ branch, and the Q4_K MMQ (block dots bit-exact, floats within
the row-L2 bound)."""
import numpy as np
import pytest
import torch

import inputs
import oracle
import q4k_pack
import bit_quantized_matmul_quantize_amd as bq
from parity_helpers import (FROB_TOL, ROW_TOL, dev_bf16, dev_u8, empty_bf16, frob_error, host_bits,
                            host_f64, rows_ok, row_error)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,k,group,seed", [(256, 512, 128, 0), (7, 96, 32, 31), (33, 512, 64, 32),
                                            (5, 1024, 256, 33), (12288, 2048, 128, 4)])
def test_dequant_bit_exact(gpu, n, k, group, seed):
    w = inputs.q2_0_weight(inputs.rng(seed), n, k, group)
    out = empty_bf16((n, k), gpu)
    bq.dequant_q2_0_to_bf16(dev_u8(w, gpu), out, n, k, group)
    assert np.array_equal(host_bits(out), oracle.dequant_q2_0_to_bf16(w, n, k, group))


# small grids take 96 x 128 tiles on 256 CUs; (1030, 5500) is large enough
# for 128 x 128 tiles, ragged in m and n
@pytest.mark.parametrize("m,n,k,seed", [(4, 256, 512, 41), (130, 200, 192, 42), (1, 1, 64, 43),
                                        (1030, 5500, 256, 44)])
def test_dense_gemm_bf16(gpu, m, n, k, seed):
    g = inputs.rng(seed)
    a = inputs.activations(g, m, k)
    wb = inputs.activations(g, n, k)
    out = empty_bf16((m, n), gpu)
    bq.dense_gemm_bf16(dev_bf16(a, gpu), dev_bf16(wb, gpu), out, m, n, k)
    # large m: sampled rows, including both sides of tile boundaries and the last row
    rows = np.arange(m) if m <= 256 else np.array([0, 127, 128, 700, 1023, 1024, m - 1])
    R = oracle.dense_gemm_bf16(np.ascontiguousarray(a[rows]), wb, len(rows), n, k)
    # fp32 accumulation and one bf16 rounding of each output
    assert rows_ok(host_f64(out)[rows], R)


def test_dense_gemm_layouts_agree(gpu):
    # the first 130 rows of an m = 1030 product (128 x 128 tiles) equal an
    # m = 130 product (96 x 128 tiles) bit for bit: each output is summed over
    # k in the same order by both layouts
    n, k = 5500, 256
    g = inputs.rng(45)
    a = inputs.activations(g, 1030, k)
    wd = dev_bf16(inputs.activations(g, n, k), gpu)
    big, small = empty_bf16((1030, n), gpu), empty_bf16((130, n), gpu)
    bq.dense_gemm_bf16(dev_bf16(a, gpu), wd, big, 1030, n, k)
    bq.dense_gemm_bf16(dev_bf16(np.ascontiguousarray(a[:130]), gpu), wd, small, 130, n, k)
    assert np.array_equal(host_bits(small), host_bits(big)[:130])


def _prefill(gpu, act, w, m, n, k, group, use_mmq):
    out = empty_bf16((m, n), gpu)
    scratch = torch.empty((n * k,), dtype=torch.bfloat16, device=gpu)
    q8 = torch.empty((bq.q8_1_act_bytes(m, k),), dtype=torch.uint8, device=gpu)
    bq.q2_0_prefill_gemm(dev_bf16(act, gpu), dev_u8(w, gpu), out, scratch, q8, m, n, k, group, use_mmq)
    return host_f64(out), q8


def test_prefill_dispatch_tiny(gpu):
    d = inputs.tiny()
    m, n, k = d["m"], d["n"], d["k"]
    R_plain = oracle.q2_0_gemv(d["act"], d["w"], m, n, k)  # unquantized bf16 input
    y_fb, _ = _prefill(gpu, d["act"], d["w"], m, n, k, 128, False)
    assert frob_error(y_fb, R_plain) <= FROB_TOL
    y_mmq, q8 = _prefill(gpu, d["act"], d["w"], m, n, k, 128, True)
    q8_ref, _ = oracle.quantize_act_q8_1(d["act"], m, k)
    torch.cuda.synchronize()
    assert np.array_equal(q8.cpu().numpy(), q8_ref)
    assert row_error(y_mmq, oracle.q2_0_mmq(q8_ref, d["w"], m, n, k)) <= ROW_TOL


def test_prefill_fallback_other_group(gpu):
    # group 64 has no MMQ path: the dispatcher takes the dequant branch even with use_mmq
    m, n, k = 9, 100, 512
    g = inputs.rng(44)
    w = inputs.q2_0_weight(g, n, k, 64)
    act = inputs.activations(g, m, k, outliers=True)
    y, _ = _prefill(gpu, act, w, m, n, k, 64, True)
    W = oracle.q2_0_decode(w, n, k, 64)
    R = inputs.bf16_bits_to_f32(act).astype(np.float64) @ W.T
    assert frob_error(y, R) <= FROB_TOL


@pytest.mark.parametrize("m", [512, 2048])
def test_prefill_fallback_qkvz(gpu, m):
    # the dispatcher's dequant branch at both prefill sizes, on 16 sampled rows
    # including the first and the last
    d = inputs.prefill_qkvz()
    n, k = d["n"], d["k"]
    act = d["act"][:m]
    y, _ = _prefill(gpu, act, d["w"], m, n, k, 128, False)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, m - 1], inputs.rng(97).choice(m, 11, replace=False)]))
    R = oracle.q2_0_gemv(np.ascontiguousarray(act[rows]), d["w"], len(rows), n, k)
    assert frob_error(y[rows], R) <= FROB_TOL


def _q4k_rows(w, n, k, r0, rt):
    return w.reshape(n, k // 256 * 144)[r0:r0 + rt].reshape(-1)


def _q8_rows(q8, m, k, rows):
    kp = (k + 255) // 256 * 256
    codes = q8[: m * kp].reshape(m, kp)[rows]
    ds = q8[m * kp:].reshape(m, kp // 32 * 4)[rows]
    return np.concatenate([codes.reshape(-1), ds.reshape(-1)])


@pytest.mark.parametrize("m,n,k,seed", [(4, 256, 512, 51), (130, 200, 768, 52), (1, 3, 256, 53)])
def test_q4k_small(gpu, m, n, k, seed):
    g = inputs.rng(seed)
    w = inputs.q4k_weight(g, n, k)
    act = inputs.activations(g, m, k, outliers=True)
    q8, _ = oracle.quantize_act_q8_1(act, m, k)
    q8d, wd = dev_u8(q8, gpu), dev_u8(w, gpu)
    out = empty_bf16((m, n), gpu)
    bq.q4k_mmq_gemm(q8d, wd, out, m, n, k)
    R = oracle.q4k_mmq(q8, w, m, n, k)
    y = host_f64(out)
    assert rows_ok(y, R)
    if n >= 256:
        assert row_error(y, R) <= ROW_TOL
    dots = torch.full((m * n * (k // 32),), -7, dtype=torch.int32, device=gpu)
    bq.q4k_mmq_blockdots(q8d, wd, dots, 0, m, 0, n, m, n, k)
    torch.cuda.synchronize()
    assert np.array_equal(dots.cpu().numpy().reshape(m, n, k // 32), oracle.q4k_blockdots(q8, w, m, n, k))


@pytest.mark.parametrize("m,n,k,seed", [(130, 300, 512, 55), (4, 256, 768, 56)])
def test_q4k_large_scales(gpu, m, n, k, seed):
    # super-block scales far above the workloads': dmin up to 6e4, so that
    # dmin * m_j (m_j up to 63) lies outside the binary16 range; the min term
    # must come from exact products in fp32 and stay finite and within bound
    g = inputs.rng(seed)
    w = inputs.q4k_weight(g, n, k).reshape(-1, 144).copy()
    nsb = w.shape[0]
    d = g.uniform(500.0, 5000.0, nsb).astype(np.float16)
    dmin = g.uniform(1100.0, 60000.0, nsb).astype(np.float16)
    w[:, 0:2] = d.view(np.uint8).reshape(nsb, 2)
    w[:, 2:4] = dmin.view(np.uint8).reshape(nsb, 2)
    w = w.reshape(-1)
    act = inputs.activations(g, m, k, outliers=True)
    q8, _ = oracle.quantize_act_q8_1(act, m, k)
    out = empty_bf16((m, n), gpu)
    bq.q4k_mmq_gemm(dev_u8(q8, gpu), dev_u8(w, gpu), out, m, n, k)
    y = host_f64(out)
    R = oracle.q4k_mmq(q8, w, m, n, k)
    assert np.all(np.isfinite(y))
    assert row_error(y, R) <= ROW_TOL


def _q4k_rows(w, n, k, r0, rt):
    """Q4_K bytes of weight rows [r0, r0+rt) (whole rows of super-blocks)."""
    return w.reshape(n, k // 256 * 144)[r0:r0 + rt].reshape(-1)


def test_q4k_ffn_prefill_sampled(gpu):
    # m = 4096 FFN gate projection [17408, 5120] in Q4_K and the down
    # projection [5120, 17408] on its own input: 16 sampled rows (first, last,
    # both sides of the middle, random) and the block dots of two 32 x 32
    # windows (first tile corner, last rows/columns)
    d = inputs.prefill_ffn(formats=("q4k",))
    H, I = d["hidden"], d["inter"]
    m = 4096
    rows = np.unique(np.concatenate([[0, 1, 2047, 2048, 4095], inputs.rng(96).choice(m, 11, replace=False)]))
    for w, n, k, act in [(d["q4k"]["wg"], I, H, d["act"]),
                         (d["q4k"]["wd"], H, I, inputs.activations(inputs.rng(54), m, I))]:
        print(f"case n={n} k={k} m={m}", flush=True)
        q8, _ = oracle.quantize_act_q8_1(act, m, k)
        q8d, wd = dev_u8(q8, gpu), dev_u8(w, gpu)
        out = empty_bf16((m, n), gpu)
        bq.q4k_mmq_gemm(q8d, wd, out, m, n, k)
        y = host_f64(out)
        R = oracle.q4k_mmq(_q8_rows(q8, m, k, rows), w, len(rows), n, k)
        assert row_error(y[rows], R) <= ROW_TOL
        for (m0, n0) in [(0, 0), (m - 32, n - 32)]:
            dots = torch.full((32 * 32 * (k // 32),), -7, dtype=torch.int32, device=gpu)
            bq.q4k_mmq_blockdots(q8d, wd, dots, m0, 32, n0, 32, m, n, k)
            torch.cuda.synchronize()
            Dref = oracle.q4k_blockdots(_q8_rows(q8, m, k, np.arange(m0, m0 + 32)), _q4k_rows(w, n, k, n0, 32),
                                        32, 32, k)
            assert np.array_equal(dots.cpu().numpy().reshape(32, 32, k // 32), Dref)


def test_q4k_strided_output(gpu):
    # q4k_mmq_gemm_ldc: same values as q4k_mmq_gemm, written into a column range
    # of a wider buffer, the other columns untouched
    m, n, k, ldc, off = 130, 200, 512, 520, 264
    g = inputs.rng(54)
    w = inputs.q4k_weight(g, n, k)
    act = inputs.activations(g, m, k)
    q8, _ = oracle.quantize_act_q8_1(act, m, k)
    q8d, wd = dev_u8(q8, gpu), dev_u8(w, gpu)
    ref = empty_bf16((m, n), gpu)
    bq.q4k_mmq_gemm(q8d, wd, ref, m, n, k)
    big = torch.full((m, ldc), -3.0, dtype=torch.bfloat16, device=gpu)
    bq.q4k_mmq_gemm_ldc(q8d, wd, big[:, off:off + n], m, n, k, ldc)
    torch.cuda.synchronize()
    assert torch.equal(big[:, off:off + n].contiguous().view(torch.int16), ref.view(torch.int16))
    mask = torch.ones_like(big, dtype=torch.bool)
    mask[:, off:off + n] = False
    assert bool((big[mask] == -3.0).all())


def _zero_subblocks(w, n, k, subs):
    """Q4_K bytes with sub-blocks `subs` of every super-block zeroed (codes 0 and m_j = 0),
    so their dequantized weights are exactly 0; the rest unchanged."""
    b = w.reshape(n * (k // 256), 144).copy()
    for j in subs:
        t, hi_nib = j // 2, j % 2
        code = b[:, 16 + 32 * t:48 + 32 * t]
        code &= np.uint8(0x0F if hi_nib else 0xF0)
        if j < 4:
            b[:, 8 + j] &= np.uint8(0xC0)               # m_j: low six bits of S[j+4]
        else:
            b[:, 8 + j] &= np.uint8(0x0F)               # low four bits of m_j: high nibble of S[j+4]
            b[:, 4 + j] &= np.uint8(0x3F)               # high two bits of m_j: top of S[j]
    return b.reshape(-1)


@pytest.mark.parametrize("m,n,k,seed", [(130, 1000, 512, 57), (260, 2100, 768, 58)])
def test_q4k_wide_activation_scale_spans(gpu, m, n, k, seed):
    # Rows whose q8_1 block scales span 2^6..2^24 inside each super-block: one
    # block per super-block holds a single value of 2000 and the others sit
    # about 2^s below; the weights under that block are exactly zero, so the
    # outputs come from the small blocks alone (the case in which the matrix
    # core's binary16 activation operand could lose them).
    g = inputs.rng(seed)
    w = _zero_subblocks(inputs.q4k_weight(g, n, k), n, k, (0, 5))
    deq = q4k_pack.dequant(w, n, k).reshape(n, k // 256, 256)
    assert np.all(deq[:, :, 0:32] == 0) and np.all(deq[:, :, 160:192] == 0)
    x = g.standard_normal((m, k)).astype(np.float32)
    wide = []
    r = 0
    for s in (6, 12, 20, 24):
        for dom in (0, 5):
            row = g.standard_normal(k).astype(np.float32) * np.float32(2000.0 * 2.0 ** -s / 2.5)
            for sb in range(k // 256):
                blk = row[256 * sb + 32 * dom:256 * sb + 32 * dom + 32]
                blk[:] = 0.0
                blk[7] = 2000.0
            x[r] = row
            wide.append(r)
            r += 3
    act = inputs.f32_to_bf16_bits(x)
    q8, _ = oracle.quantize_act_q8_1(act, m, k)
    kp = (k + 255) // 256 * 256
    d = q8[m * kp:].copy().view(np.uint16).reshape(m, kp // 32, 2)[:, :, 0].copy().view(np.float16).astype(np.float64)
    assert max(d[i][d[i] > 0].max() / d[i][d[i] > 0].min() for i in wide) >= 2.0 ** 22
    out = empty_bf16((m, n), gpu)
    bq.q4k_mmq_gemm(dev_u8(q8, gpu), dev_u8(w, gpu), out, m, n, k)
    y = host_f64(out)
    rows = np.unique(np.concatenate([wide, [1, 2, m - 1], inputs.rng(seed).choice(m, 6, replace=False)]))
    R = oracle.q4k_mmq(_q8_rows(q8, m, k, rows), w, len(rows), n, k)
    assert np.all(np.linalg.norm(R, axis=1) > 0)
    assert row_error(y[rows], R) <= ROW_TOL

"""GPU parity: Q2_0 MMQ.  Integer block dots bit-exact (through the same
kernel path, dumped before the epilogue); bf16 outputs within the row-L2
bound of the oracle's fp64 result."""
import numpy as np
import pytest
import torch

import inputs
import oracle
import bit_quantized_matmul_quantize_amd as bq
from parity_helpers import ROW_TOL, dev_bf16, dev_u8, empty_bf16, host_f64, rows_ok, row_error

pytestmark = pytest.mark.gpu


def _q8_dev(gpu, act, m, k):
    q8, _ = oracle.quantize_act_q8_1(act, m, k)  # bit-exact with the device quantizer (tested)
    return q8, dev_u8(q8, gpu)


def _mmq(gpu, q8d, wd, m, n, k):
    out = empty_bf16((m, n), gpu)
    bq.q2_0_mmq_gemm(q8d, wd, out, m, n, k)
    return host_f64(out)


def _dots(gpu, q8d, wd, m0, mt, n0, nt, m, n, k):
    out = torch.full((mt * nt * (k // 32),), -7, dtype=torch.int32, device=gpu)
    bq.q2_0_mmq_blockdots(q8d, wd, out, m0, mt, n0, nt, m, n, k)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(mt, nt, k // 32)


def test_tiny_full(gpu):
    d = inputs.tiny()
    m, n, k = d["m"], d["n"], d["k"]
    q8, q8d = _q8_dev(gpu, d["act"], m, k)
    wd = dev_u8(d["w"], gpu)
    R = oracle.q2_0_mmq(q8, d["w"], m, n, k)
    assert row_error(_mmq(gpu, q8d, wd, m, n, k), R) <= ROW_TOL
    D = _dots(gpu, q8d, wd, 0, m, 0, n, m, n, k)
    assert np.array_equal(D, oracle.q2_0_blockdots(q8, d["w"], m, n, k))


@pytest.mark.parametrize("m,n,k,seed", [
    (130, 200, 384, 11),   # ragged m and n over several tiles, 3 groups
    (1, 1, 128, 12),       # degenerate single output
    (257, 131, 1024, 13),  # tails on both sides, n % 4 != 0 (scalar stores)
    (64, 384, 2048, 14),
])
def test_ragged_shapes(gpu, m, n, k, seed):
    g = inputs.rng(seed)
    w = inputs.q2_0_weight(g, n, k)
    act = inputs.activations(g, m, k, outliers=True)
    q8, q8d = _q8_dev(gpu, act, m, k)
    wd = dev_u8(w, gpu)
    R = oracle.q2_0_mmq(q8, w, m, n, k)
    assert rows_ok(_mmq(gpu, q8d, wd, m, n, k), R)
    mt, nt = min(m, 40), min(n, 70)
    m0, n0 = m - mt, n - nt
    D = _dots(gpu, q8d, wd, m0, mt, n0, nt, m, n, k)
    Dref = oracle.q2_0_blockdots(_rows_q8(q8, m, k, m0, mt), w, mt, n, k)
    assert np.array_equal(D, Dref[:, n0:n0 + nt])


def _rows_q8(q8, m, k, r0, rt):
    """q8_1 buffer of rows [r0, r0+rt) of an m-row buffer (layout-level copy)."""
    kp = (k + 255) // 256 * 256
    codes = q8[: m * kp].reshape(m, kp)[r0:r0 + rt]
    ds = q8[m * kp:].reshape(m, kp // 32 * 4)[r0:r0 + rt]
    return np.concatenate([codes.reshape(-1), ds.reshape(-1)])


def test_integer_case_exact(gpu):
    # amax 127 per block -> d = 1, q = x; weight scales 1 -> exact small integers
    m, n, k = 33, 65, 256
    g = inputs.rng(15)
    x = g.integers(-3, 4, size=(m, k)).astype(np.float32)
    x[:, ::32] = 127
    x[:, 1::32] = -127
    act = inputs.f32_to_bf16_bits(x)
    codes = inputs.q2_0_weight(g, n, k)
    w = codes.copy()
    w[n * k // 4:] = np.frombuffer(np.ones(n * k // 128, np.float16).tobytes(), np.uint8)
    q8, q8d = _q8_dev(gpu, act, m, k)
    R = oracle.q2_0_mmq(q8, w, m, n, k)
    assert np.all(R == np.round(R))
    y = _mmq(gpu, q8d, dev_u8(w, gpu), m, n, k)
    small = np.abs(R) <= 256
    assert np.array_equal(y[small], R[small])


@pytest.mark.parametrize("m", [512, 2048])
def test_prefill_qkvz_sampled(gpu, m):
    d = inputs.prefill_qkvz()
    n, k = d["n"], d["k"]
    act = d["act"][:m]
    q8, q8d = _q8_dev(gpu, act, m, k)
    wd = dev_u8(d["w"], gpu)
    y = _mmq(gpu, q8d, wd, m, n, k)
    rows = np.unique(np.concatenate([[0, m - 1], inputs.rng(99).choice(m, 14, replace=False)]))
    R = oracle.q2_0_mmq(_rows_sel(q8, m, k, rows), d["w"], len(rows), n, k)
    assert row_error(y[rows], R) <= ROW_TOL
    # block dots on two windows (first tile corner and the last rows/columns)
    for (m0, n0) in [(0, 0), (m - 32, n - 32)]:
        D = _dots(gpu, q8d, wd, m0, 32, n0, 32, m, n, k)
        Dref = oracle.q2_0_blockdots(_rows_q8(q8, m, k, m0, 32), _w_rows(d["w"], n, k, n0, 32), 32, 32, k)
        assert np.array_equal(D, Dref)


def test_large_grid_ragged(gpu):
    # a grid large enough for the 128 x 128 tile (the small shapes above take
    # 96 x 128 tiles), ragged in m and n, on sampled rows incl. the last tile
    m, n, k = 1030, 5500, 256
    g = inputs.rng(16)
    w = inputs.q2_0_weight(g, n, k)
    act = inputs.activations(g, m, k, outliers=True)
    q8, q8d = _q8_dev(gpu, act, m, k)
    y = _mmq(gpu, q8d, dev_u8(w, gpu), m, n, k)
    rows = np.array([0, 127, 128, 700, 1023, 1024, 1029])
    R = oracle.q2_0_mmq(_rows_sel(q8, m, k, rows), w, len(rows), n, k)
    assert rows_ok(y[rows], R)


def _w_rows(w, n, k, r0, rt):
    """Q2_0 bytes of weight rows [r0, r0+rt) (layout-level copy, group 128)."""
    codes = w[: n * k // 4].reshape(n, k // 4)[r0:r0 + rt]
    sc = w[n * k // 4:].reshape(n, k // 128 * 2)[r0:r0 + rt]
    return np.concatenate([codes.reshape(-1), sc.reshape(-1)])


def _rows_sel(q8, m, k, rows):
    kp = (k + 255) // 256 * 256
    codes = q8[: m * kp].reshape(m, kp)[rows]
    ds = q8[m * kp:].reshape(m, kp // 32 * 4)[rows]
    return np.concatenate([codes.reshape(-1), ds.reshape(-1)])


def test_batch_invariance(gpu):
    # rows shared by the m = 512 and m = 2048 runs give identical outputs (the
    # two runs use different tile shapes, 96 x 128 and 128 x 128 on 256 CUs:
    # each output is folded in the same order by both)
    d = inputs.prefill_qkvz()
    n, k = d["n"], d["k"]
    wd = dev_u8(d["w"], gpu)
    q8a, q8ad = _q8_dev(gpu, d["act"][:512], 512, k)
    q8b, q8bd = _q8_dev(gpu, d["act"], 2048, k)
    ya = _mmq(gpu, q8ad, wd, 512, n, k)
    yb = _mmq(gpu, q8bd, wd, 2048, n, k)
    assert np.array_equal(ya, yb[:512])


def test_ffn_prefill_q2_sampled(gpu):
    # m = 4096 FFN prefill in Q2_0: gate [17408, 5120] and down [5120, 17408],
    # 16 sampled rows (first, last, both sides of the middle, random) and the
    # block dots of two 32 x 32 windows (first tile corner, last rows/columns)
    d = inputs.prefill_ffn(formats=("q2_0",))
    H, I, m = d["hidden"], d["inter"], 4096
    rows = np.unique(np.concatenate([[0, 1, 2047, 2048, 4095], inputs.rng(97).choice(m, 11, replace=False)]))
    for w, n, k, act in [(d["q2"]["wg"], I, H, d["act"]),
                         (d["q2"]["wd"], H, I, inputs.activations(inputs.rng(55), m, I))]:
        print(f"case n={n} k={k} m={m}", flush=True)
        q8, q8d = _q8_dev(gpu, act, m, k)
        wd = dev_u8(w, gpu)
        y = _mmq(gpu, q8d, wd, m, n, k)
        R = oracle.q2_0_mmq(_rows_sel(q8, m, k, rows), w, len(rows), n, k)
        assert row_error(y[rows], R) <= ROW_TOL
        for (m0, n0) in [(0, 0), (m - 32, n - 32)]:
            D = _dots(gpu, q8d, wd, m0, 32, n0, 32, m, n, k)
            Dref = oracle.q2_0_blockdots(_rows_q8(q8, m, k, m0, 32), _w_rows(w, n, k, n0, 32), 32, 32, k)
            assert np.array_equal(D, Dref)


@pytest.mark.parametrize("m,n,k,ldc,off,seed", [(300, 136, 512, 1024, 256, 60),    # ragged tiles
                                                (130, 256, 1024, 266, 8, 61),    # ldc % 4 != 0: scalar stores
                                                (64, 128, 384, 128, 0, 62)])     # ldc == n
def test_strided_output(gpu, m, n, k, ldc, off, seed):
    # q2_0_mmq_gemm_ldc writes the same values as q2_0_mmq_gemm into columns
    # [off, off + n) of a buffer with row stride ldc and leaves the rest alone
    # (off % 8 == 0 keeps the first element 16-byte aligned)
    g = inputs.rng(seed)
    w = inputs.q2_0_weight(g, n, k)
    act = inputs.activations(g, m, k, outliers=True)
    _, q8d = _q8_dev(gpu, act, m, k)
    wd = dev_u8(w, gpu)
    ref = empty_bf16((m, n), gpu)
    bq.q2_0_mmq_gemm(q8d, wd, ref, m, n, k)
    big = torch.full((m, ldc), -3.0, dtype=torch.bfloat16, device=gpu)
    bq.q2_0_mmq_gemm_ldc(q8d, wd, big[:, off:off + n], m, n, k, ldc)
    torch.cuda.synchronize()
    got = big[:, off:off + n].contiguous()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    mask = torch.ones_like(big, dtype=torch.bool)
    mask[:, off:off + n] = False
    assert bool((big[mask] == -3.0).all())


# ---- rows whose q8_1 block scales span far more than the integer fold's 2^5 ----

def _wide_span_case(m, n, k, seed, spans):
    """Activations where some rows hold one dominant block (a single value of
    2000 in a block of zeros) and small blocks whose scales sit about 2^s
    below it, for s in `spans`; the dominant blocks sit at block 0 (sharing a
    128-group with small blocks) or block 4 (a group of its own), and every
    weight row has code 2 (weight 0) under both, so those rows' products come
    from the small blocks alone.  Other rows are ordinary N(0,1) activations
    with outlier channels."""
    g = inputs.rng(seed)
    x = g.standard_normal((m, k)).astype(np.float32)
    x[:, g.choice(k, max(1, k // 100), replace=False)] *= 20.0
    wide_rows = []
    r = 0
    for s in spans:
        for dom in (0, 4):
            row = g.standard_normal(k).astype(np.float32) * np.float32(2000.0 * 2.0 ** -s / 2.5)
            row[32 * dom:32 * dom + 32] = 0.0
            row[32 * dom + 7] = 2000.0
            x[r] = row
            wide_rows.append(r)
            r += 3  # spread the wide rows over the first tile, with ordinary rows between
    act = inputs.f32_to_bf16_bits(x)
    w = inputs.q2_0_weight(g, n, k)
    codes = w[: n * k // 4].reshape(n, k // 4)
    # byte t of group 0 holds k-offsets t, t+32, t+64, t+96 in bit fields 0..3:
    # field 0 of group 0 is block 0, field 0 of group 1 is block 4
    for grp in (0, 1):
        b = codes[:, 32 * grp:32 * grp + 32]
        b &= np.uint8(0xFC)
        b |= np.uint8(0x02)
    return act, w, np.array(wide_rows)


@pytest.mark.parametrize("m,n,k,seed", [(130, 384, 1024, 17),     # 96 x 128 tiles, one tile with wide rows
                                        (1030, 5500, 512, 18)])   # 128 x 128 tiles
def test_fold_wide_block_scale_spans(gpu, m, n, k, seed):
    act, w, wide = _wide_span_case(m, n, k, seed, spans=(6, 12, 20, 24))
    q8, q8d = _q8_dev(gpu, act, m, k)
    _, ds = _planes(q8, m, k)
    d = ds[:, :, 0].copy().view(np.float16).astype(np.float64)  # block scales
    for r in wide:  # the spans asked for are really there
        nz = d[r][d[r] > 0]
        assert nz.max() / nz.min() >= 2.0 ** 5
    assert max(d[r][d[r] > 0].max() / d[r][d[r] > 0].min() for r in wide) >= 2.0 ** 20
    y = _mmq(gpu, q8d, dev_u8(w, gpu), m, n, k)
    rows = np.unique(np.concatenate([wide, [1, 2, 127, 128, m - 1], inputs.rng(seed).choice(m, 6, replace=False)]))
    R = oracle.q2_0_mmq(_rows_sel(q8, m, k, rows), w, len(rows), n, k)
    # the dominant blocks contribute nothing: every product comes from the small blocks
    assert np.all(np.linalg.norm(R[np.isin(rows, wide)], axis=1) > 0)
    assert row_error(y[rows], R) <= ROW_TOL
    # the block dots of a window over the wide rows are still exact
    D = _dots(gpu, q8d, dev_u8(w, gpu), 0, 32, n - 40, 40, m, n, k)
    Dref = oracle.q2_0_blockdots(_rows_q8(q8, m, k, 0, 32), _w_rows(w, n, k, n - 40, 40), 32, 40, k)
    assert np.array_equal(D, Dref)


def _planes(q8, m, k):
    """codes [m][kpad] (int8 bytes) and the (d, s) bit pairs [m][kpad/32][2]."""
    kp = (k + 255) // 256 * 256
    return q8[: m * kp].reshape(m, kp), q8[m * kp:].copy().view(np.uint16).reshape(m, kp // 32, 2)


def test_fold_wide_span_rows_do_not_change_other_tiles(gpu):
    # an m-tile of ordinary rows gives the same bits whether or not another
    # tile of the same call holds wide rows (tiles fold independently)
    m, n, k = 256, 384, 1024
    act, w, _ = _wide_span_case(m, n, k, 19, spans=(20,))
    plain = act.copy()
    plain[:128] = inputs.activations(inputs.rng(20), 128, k)
    q8a, q8ad = _q8_dev(gpu, act, m, k)
    q8b, q8bd = _q8_dev(gpu, plain, m, k)
    wd = dev_u8(w, gpu)
    assert np.array_equal(_mmq(gpu, q8ad, wd, m, n, k)[128:], _mmq(gpu, q8bd, wd, m, n, k)[128:])


def _subnormal_scale_case(m, n, k, seed):
    """Rows whose one dominant block sets the row's largest q8_1 scale to
    binary16 exponent field 6, 7 or 8 (a single value of 0.375, 0.75 or 1.5)
    while every other block holds values whose scale is subnormal, d = j·2^-24
    for j in 1..9 (block maximum 127·j·2^-24); every weight row has code 2
    under the dominant block, so those rows' products come from the
    subnormal-scale blocks alone.  Other rows are ordinary N(0,1) activations
    with outlier channels."""
    g = inputs.rng(seed)
    x = g.standard_normal((m, k)).astype(np.float32)
    x[:, g.choice(k, max(1, k // 100), replace=False)] *= 20.0
    rows = []
    for i, top in enumerate((0.375, 0.75, 1.5) * 2):
        r = 3 * i
        row = np.zeros(k, dtype=np.float32)
        for b in range(1, k // 32):
            amax = np.float32(127.0 * int(g.integers(1, 10)) * 2.0 ** -24)
            vals = (g.uniform(-1.0, 1.0, 32) * amax).astype(np.float32)
            vals[int(g.integers(0, 32))] = amax if g.random() < 0.5 else -amax
            row[32 * b:32 * b + 32] = vals
        row[7] = top
        x[r] = row
        rows.append(r)
    act = inputs.f32_to_bf16_bits(x)
    w = inputs.q2_0_weight(g, n, k)
    codes = w[: n * k // 4].reshape(n, k // 4)
    b = codes[:, 0:32]  # field 0 of group 0 is block 0
    b &= np.uint8(0xFC)
    b |= np.uint8(0x02)
    return act, w, np.array(rows)


@pytest.mark.parametrize("m,n,k,seed", [(130, 384, 1024, 21),     # 96 x 128 tiles
                                        (1030, 5500, 512, 22)])   # 128 x 128 tiles
def test_fold_subnormal_block_scales(gpu, m, n, k, seed):
    # subnormal q8_1 scales are applied exactly next to a row maximum of any
    # exponent (field 7 puts them at the bottom of the top band's reach)
    act, w, sub = _subnormal_scale_case(m, n, k, seed)
    q8, q8d = _q8_dev(gpu, act, m, k)
    _, ds = _planes(q8, m, k)
    fields = (ds[:, :, 0] >> 10) & 31
    for r in sub:  # the scales asked for are really there
        assert fields[r, 0] in (6, 7, 8) and np.all(fields[r, 1:k // 32] == 0)
        assert np.all(ds[r, 1:k // 32, 0] > 0)
    assert 7 in {int(fields[r, 0]) for r in sub}
    y = _mmq(gpu, q8d, dev_u8(w, gpu), m, n, k)
    rows = np.unique(np.concatenate([sub, [1, 2, 127, 128, m - 1]]))
    R = oracle.q2_0_mmq(_rows_sel(q8, m, k, rows), w, len(rows), n, k)
    assert np.all(np.linalg.norm(R[np.isin(rows, sub)], axis=1) > 0)
    assert row_error(y[rows], R) <= ROW_TOL

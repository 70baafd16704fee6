"""GPU parity: the m = 4096 FFN prefill chain in both weight formats, as the
bench runs it -- quantize_act_q8_1 of x, gate and up MMQ sharing that q8_1
input, silu_mul_quantize_q8_1 of (gate, up), down MMQ on the device's own
q8_1 of h -- checked stage by stage (each stage against the oracle on the
device's previous output) and end to end (the oracle's own chain, with the
bf16 roundings and the re-quantization at the same points).

[page layers/ops/q4k_mmq.rs, module doc: each prefill quantizes its
 activations to q8_1 and runs the GEMM with a BF16 store; page
 layers/dense_ffn_decode_batch.rs, fn forward_km_q2: gate, up, silu_mul into
 the gate buffer, down.]"""
import numpy as np
import pytest
import torch

import inputs
import oracle
import bit_quantized_matmul_quantize_amd as bq
from parity_helpers import (ROW_TOL, bf16_ulp_distance, dev_bf16, dev_u8, empty_bf16, host_bits, host_f64,
                            row_error)

pytestmark = pytest.mark.gpu

M, H, I = 4096, inputs.HIDDEN, inputs.INTER


@pytest.fixture(scope="module")
def ffn():
    return inputs.prefill_ffn()


def _rows_q8(q8, m, k, rows):
    """q8_1 buffer of the selected rows of an m-row buffer (layout-level copy)."""
    kp = (k + 255) // 256 * 256
    codes = q8[: m * kp].reshape(m, kp)[rows]
    ds = q8[m * kp:].reshape(m, kp // 32 * 4)[rows]
    return np.concatenate([codes.reshape(-1), ds.reshape(-1)])


def _log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("fmt", ["q2_0", "q4k"])
def test_ffn_prefill_chain(gpu, ffn, fmt):
    key, gemm, omm = {"q2_0": ("q2", bq.q2_0_mmq_gemm, oracle.q2_0_mmq),
                      "q4k": ("q4k", bq.q4k_mmq_gemm, oracle.q4k_mmq)}[fmt]
    wg, wu, wd = (ffn[key][name] for name in ("wg", "wu", "wd"))
    x = ffn["act"]
    _log(f"ffn chain {fmt}: m={M} hidden={H} inter={I}")
    wgd, wud, wdd = dev_u8(wg, gpu), dev_u8(wu, gpu), dev_u8(wd, gpu)
    q8a = torch.empty((bq.q8_1_act_bytes(M, H),), dtype=torch.uint8, device=gpu)
    q8h = torch.empty((bq.q8_1_act_bytes(M, I),), dtype=torch.uint8, device=gpu)
    gate, up, out = empty_bf16((M, I), gpu), empty_bf16((M, I), gpu), empty_bf16((M, H), gpu)
    bq.quantize_act_q8_1(dev_bf16(x, gpu), q8a, M, H)
    gemm(q8a, wgd, gate, M, I, H)
    gemm(q8a, wud, up, M, I, H)
    bq.silu_mul_quantize_q8_1(gate, up, q8h, M, I)
    gemm(q8h, wdd, out, M, H, I)
    # the device's h, from the unfused silu_mul on the same gate and up: the
    # fused quantizer's input (the two are equal bit for bit, tested apart)
    h = empty_bf16((M, I), gpu)
    bq.silu_mul_bf16(gate, up, h, M * I)
    torch.cuda.synchronize()
    q8a_dev, q8h_dev = q8a.cpu().numpy(), q8h.cpu().numpy()
    g_bits, u_bits, h_bits = host_bits(gate), host_bits(up), host_bits(h)
    y = host_f64(out)
    rows = np.unique(np.concatenate([[0, 1, 2047, 2048, M - 1], inputs.rng(98).choice(M, 11, replace=False)]))

    # stage 1: q8_1 of x, whole buffer, bit-exact
    q8a_ref, flagged = oracle.quantize_act_q8_1(x, M, H)
    assert flagged == 0 and np.array_equal(q8a_dev, q8a_ref)
    _log("stage 1 (quantize x) bit-exact")
    # stage 2: gate and up on the sampled rows, from the device's q8_1 of x
    q8a_rows = _rows_q8(q8a_dev, M, H, rows)
    Rg = omm(q8a_rows, wg, len(rows), I, H)
    Ru = omm(q8a_rows, wu, len(rows), I, H)
    eg = row_error(inputs.bf16_bits_to_f32(g_bits[rows]).astype(np.float64), Rg)
    eu = row_error(inputs.bf16_bits_to_f32(u_bits[rows]).astype(np.float64), Ru)
    _log(f"stage 2 (gate, up) row errors {eg:.2e} {eu:.2e}")
    assert eg <= ROW_TOL and eu <= ROW_TOL
    # stage 3: h = silu(gate) * up on the device's gate and up, every element
    # within one bf16 step of the oracle; the q8_1 of h from the fused
    # producer equals the oracle's quantization of the device's h, whole buffer
    assert bf16_ulp_distance(h_bits, oracle.silu_mul_bf16(g_bits, u_bits)).max() <= 1
    q8h_ref, flagged = oracle.quantize_act_q8_1(h_bits, M, I)
    assert flagged == 0 and np.array_equal(q8h_dev, q8h_ref)
    _log("stage 3 (silu_mul, quantize h) bit-exact on the device's h")
    # stage 4: down on the sampled rows, from the device's own q8_1 of h
    Rd = omm(_rows_q8(q8h_dev, M, I, rows), wd, len(rows), H, I)
    ed = row_error(y[rows], Rd)
    _log(f"stage 4 (down) row error {ed:.2e}")
    assert ed <= ROW_TOL
    # end to end: the oracle's chain from x on the same rows (gate and up
    # rounded to bf16, silu_mul, re-quantized, down)
    h_o = oracle.silu_mul_bf16(oracle.round_bf16(Rg), oracle.round_bf16(Ru))
    q8h_o, flagged = oracle.quantize_act_q8_1(h_o, len(rows), I)
    assert flagged == 0
    Rend = omm(q8h_o, wd, len(rows), H, I)
    ee = row_error(y[rows], Rend)
    _log(f"end to end row error {ee:.2e}")
    assert ee <= ROW_TOL

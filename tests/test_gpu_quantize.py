"""GPU parity: quantize_act_q8_1 against the oracle, bit-exact over the whole
q8_1 buffer (codes, d and s)."""
import numpy as np
import pytest
import torch

import inputs
import oracle
import bit_quantized_matmul_quantize_amd as bq
from parity_helpers import dev_bf16, dev_u8

pytestmark = pytest.mark.gpu


def _run(gpu, act, m, k):
    out = torch.full((bq.q8_1_act_bytes(m, k),), 0x5A, dtype=torch.uint8, device=gpu)
    bq.quantize_act_q8_1(dev_bf16(act, gpu), out, m, k)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("m,k,outliers,seed", [
    (4, 512, False, 0),        # tiny workload
    (1, 1, False, 1),          # one value, padded to 256
    (3, 300, True, 2),         # ragged k: scalar tail and padding
    (5, 2056, True, 3),        # k % 8 == 0 but not % 256: vector path then padding
    (7, 4100, False, 4),       # k % 8 != 0: scalar path
    (130, 2048, True, 5),      # more than one 2048 chunk per row? no: exactly one; 130 rows
    (2, 5120, False, 6),       # three 2048-chunks per row
])
def test_quantize_bit_exact(gpu, m, k, outliers, seed):
    act = inputs.activations(inputs.rng(seed), m, k, outliers=outliers)
    ref, flagged = oracle.quantize_act_q8_1(act, m, k)
    assert flagged == 0
    got = _run(gpu, act, m, k)
    assert np.array_equal(got, ref)


def test_quantize_edge_values(gpu):
    # zero blocks, a ties block (amax 127 -> d = 1), tiny values (subnormal d)
    m, k = 3, 256
    x = np.zeros((m, k), np.float32)
    x[1, :8] = [127.0, 2.5, -2.5, 0.5, -0.5, 126.5, -1.5, 3.5]
    x[2] = np.linspace(-1e-6, 1e-6, k, dtype=np.float32)
    x[2, 32:64] = 3e-5
    act = inputs.f32_to_bf16_bits(x)
    ref, _ = oracle.quantize_act_q8_1(act, m, k)
    assert np.array_equal(_run(gpu, act, m, k), ref)


def _near_ties(seed, count):
    """Block maxima amax (which fix d = fp16(amax/127)) with the bf16 values x,
    |x| <= amax, whose binary32 quotient x/d lies within 2^-12 of a
    half-integer (exact ties included), where roundf's tie rule and the
    division's last bit decide the code."""
    F = np.float32
    bits = np.arange(1 << 16, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) <= 2047) & (x != 0)].astype(F)
    g = np.random.default_rng(seed)
    found = []
    while len(found) < count:
        amax = F(np.abs(g.choice(x)))
        d = F(np.float16(amax / F(127)))
        if d == 0:
            continue
        with np.errstate(over="ignore"):
            t = np.abs((x / d).astype(F))
        sel = (np.abs(x) <= amax) & (np.abs(t - np.floor(t) - F(0.5)) < F(2.0 ** -12))
        if sel.any():
            found.append((amax, x[sel]))
    return found


def test_quantize_near_ties(gpu):
    # blocks whose quotients x/d sit on or within 2^-12 of a half-integer
    rows = []
    for amax, xs in _near_ties(23, 64):
        vals = np.resize(xs, 31)
        rows.append(np.concatenate([[amax], vals * np.where(np.arange(31) % 2, -1, 1)]).astype(np.float32))
    x = np.stack(rows).reshape(8, -1)  # 8 rows of 8 blocks of 32
    m, k = x.shape
    act = inputs.f32_to_bf16_bits(x)
    ref, flagged = oracle.quantize_act_q8_1(act, m, k)
    assert flagged == 0
    assert np.array_equal(_run(gpu, act, m, k), ref)


def test_quantize_prefill_full_size(gpu):
    # m = 2048, k = 2048 qkvz prefill input (with outlier channels), whole buffer
    d = inputs.prefill_qkvz()
    act = d["act"]
    ref, _ = oracle.quantize_act_q8_1(act, 2048, 2048)
    assert np.array_equal(_run(gpu, act, 2048, 2048), ref)


def test_quantize_ffn_down_input_full_size(gpu):
    # m = 4096, k = 17408: the largest activation the FFN prefill quantizes
    g = inputs.rng(77)
    act = inputs.activations(g, 4096, 17408)
    ref, _ = oracle.quantize_act_q8_1(act, 4096, 17408)
    assert np.array_equal(_run(gpu, act, 4096, 17408), ref)


# ---- silu_mul fused into the quantizer ------------------------------------------

def _fused(gpu, gate, up, m, k):
    out = torch.full((bq.q8_1_act_bytes(m, k),), 0x5A, dtype=torch.uint8, device=gpu)
    bq.silu_mul_quantize_q8_1(dev_bf16(gate, gpu), dev_bf16(up, gpu), out, m, k)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _chain(gpu, gate, up, m, k):
    """silu_mul_bf16 then quantize_act_q8_1 on the device: the calls the fused entry replaces."""
    g, u = dev_bf16(gate, gpu), dev_bf16(up, gpu)
    h = torch.empty((m, k), dtype=torch.bfloat16, device=gpu)
    bq.silu_mul_bf16(g, u, h, m * k)
    out = torch.full((bq.q8_1_act_bytes(m, k),), 0x5A, dtype=torch.uint8, device=gpu)
    bq.quantize_act_q8_1(h, out, m, k)
    torch.cuda.synchronize()
    return out.cpu().numpy(), h


@pytest.mark.parametrize("m,k,seed", [(4, 512, 80), (3, 300, 81), (7, 4100, 82), (64, 17408, 83)])
def test_silu_mul_quantize_equals_chain(gpu, m, k, seed):
    g = inputs.rng(seed)
    gate = inputs.activations(g, m, k, outliers=True)
    up = inputs.activations(g, m, k)
    got = _fused(gpu, gate, up, m, k)
    ref, h = _chain(gpu, gate, up, m, k)
    assert np.array_equal(got, ref)
    # and against the oracle on the device's own bf16 hidden activation
    h_bits = h.view(torch.int16).cpu().numpy().view(np.uint16)
    oref, flagged = oracle.quantize_act_q8_1(h_bits, m, k)
    assert flagged == 0 and np.array_equal(got, oref)


def test_silu_mul_quantize_ffn_full_size(gpu):
    # m = 4096, k = 17408: the FFN down projection's input at prefill
    g = inputs.rng(84)
    gate = inputs.activations(g, 4096, 17408)
    up = inputs.activations(g, 4096, 17408)
    got = _fused(gpu, gate, up, 4096, 17408)
    ref, _ = _chain(gpu, gate, up, 4096, 17408)
    assert np.array_equal(got, ref)

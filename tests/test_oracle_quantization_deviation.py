"""The MMQ's deviation from the unquantized product, for information.

The prefill MMQ multiplies q8_1-quantized activations; its reference is the
product of those dequantized activations (the oracle's MMQ).  How far that
lies from the product of the original bf16 activations (the oracle's GEMV
definition, which quantizes nothing) is a property of the method, not of the
kernels: it is computed here from the oracle alone and printed, with a loose
bound that only a broken quantizer or decoder would exceed.  Workloads: the
tiny case whole and the qkvz prefill (outlier channels) on 16 rows.
[page layers/qwen3_ssm/init_q2.rs, fn qkvz_q2_prefill_gemm: the MMQ branch
 quantizes the bf16 input to q8_1; the fallback branch runs on the original
 bf16 input.]"""
import numpy as np

import inputs
import oracle
from parity_helpers import row_error


def _deviation(act, w, m, n, k):
    q8, flagged = oracle.quantize_act_q8_1(act, m, k)
    assert flagged == 0
    return row_error(oracle.q2_0_mmq(q8, w, m, n, k), oracle.q2_0_gemv(act, w, m, n, k))


def test_quantization_deviation_tiny():
    c = inputs.tiny()
    dev = _deviation(c["act"], c["w"], c["m"], c["n"], c["k"])
    print(f"tiny m=4 n=256 k=512: max |MMQ - unquantized| / row L2 = {dev:.2e}")
    assert 1e-5 < dev < 1e-2


def test_quantization_deviation_prefill_outliers():
    d = inputs.prefill_qkvz()
    m = 16
    dev = _deviation(d["act"][:m], d["w"], m, d["n"], d["k"])
    print(f"qkvz prefill, 16 rows with outlier channels: max |MMQ - unquantized| / row L2 = {dev:.2e}")
    assert 1e-5 < dev < 1e-2

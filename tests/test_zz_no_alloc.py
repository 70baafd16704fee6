"""The prefill dispatcher without a workspace argument
(q2_0_prefill_gemm_noalloc) against q2_0_prefill_gemm with caller buffers:
the same kernels on the same inputs, so the outputs are equal bit for bit.
Two calls in a row on each branch, the second smaller, since the library's
workspace array keeps the previous call's contents."""
import numpy as np
import pytest
import torch

import inputs
import bit_quantized_matmul_quantize_amd as bq
from parity_helpers import dev_bf16, dev_u8, empty_bf16, host_bits

pytestmark = pytest.mark.gpu


def _pair(gpu, act, w, m, n, k, group, use_mmq):
    a, wd = dev_bf16(act, gpu), dev_u8(w, gpu)
    ref = empty_bf16((m, n), gpu)
    scratch = torch.empty((n * k,), dtype=torch.bfloat16, device=gpu)
    q8 = torch.empty((bq.q8_1_act_bytes(m, k),), dtype=torch.uint8, device=gpu)
    bq.q2_0_prefill_gemm(a, wd, ref, scratch, q8, m, n, k, group, use_mmq)
    got = torch.full((m, n), 7.0, dtype=torch.bfloat16, device=gpu)
    bq.q2_0_prefill_gemm_noalloc(a, wd, got, m, n, k, group, use_mmq)
    return host_bits(got), host_bits(ref)


@pytest.mark.parametrize("use_mmq,group,shapes", [
    # MMQ branch: the m = 512 qkvz prefill, then a smaller ragged call
    (True, 128, [(512, 12288, 2048, 201), (130, 300, 1024, 202)]),
    # dequant branch: the qkvz weight (50 MB of bf16 workspace), then a smaller one
    (False, 128, [(256, 12288, 2048, 203), (9, 100, 512, 204)]),
    # group 64 has no MMQ path: the dequant branch even with use_mmq
    (True, 64, [(33, 1000, 1024, 205), (5, 70, 256, 206)]),
])
def test_noalloc_equals_workspace_entry(gpu, use_mmq, group, shapes):
    for m, n, k, seed in shapes:
        print(f"noalloc use_mmq={use_mmq} group={group} m={m} n={n} k={k}", flush=True)
        g = inputs.rng(seed)
        w = inputs.q2_0_weight(g, n, k, group)
        act = inputs.activations(g, m, k, outliers=True)
        got, ref = _pair(gpu, act, w, m, n, k, group, use_mmq)
        assert np.array_equal(got, ref)


def test_noalloc_rejects_oversize(gpu):
    # beyond the 64 MiB workspace: BQ_EUNSUPPORTED, nothing launched
    m, n, k = 4096, 64, 16384  # q8_1 of [4096][16384] is 72 MiB
    act = torch.zeros((m, k), dtype=torch.bfloat16, device=gpu)
    w = torch.zeros((bq.q2_0_weight_bytes(n, k, 128),), dtype=torch.uint8, device=gpu)
    out = empty_bf16((m, n), gpu)
    with pytest.raises(bq.BqmmError) as e:
        bq.q2_0_prefill_gemm_noalloc(act, w, out, m, n, k, 128, True)
    assert e.value.status == bq.BQ_EUNSUPPORTED and "workspace" in str(e.value)

"""Every entry point captured in one HIP graph, and run on two streams at once.

The timing harness replays captured graphs, and a caller may capture these
calls too.  A sequence of calls (every entry point, chained where one feeds
the next) is run eagerly, then captured and replayed three times; before each
replay the outputs are cleared with a fill kernel and unrelated eager work
runs, and after it every output must equal the eager result bit for bit.
"""
import pytest
import torch

import inputs
import bit_quantized_matmul_quantize_amd as bq
from parity_helpers import dev_bf16, dev_u8, empty_bf16

pytestmark = pytest.mark.gpu


def _u8(nbytes, gpu):
    return torch.empty((nbytes,), dtype=torch.uint8, device=gpu)


def _setup(gpu):
    g = inputs.rng(91)
    m, n, k = 256, 1024, 2048
    n4 = 512
    t = {}
    t["act"] = dev_bf16(inputs.activations(g, m, k, outliers=True), gpu)
    t["w2"] = dev_u8(inputs.q2_0_weight(g, n, k), gpu)
    t["w4"] = dev_u8(inputs.q4k_weight(g, n4, k), gpu)
    t["wbf"] = dev_bf16(inputs.bf16_weight(g, n4, k), gpu)
    t["gate"] = dev_bf16(inputs.activations(g, 8, k), gpu)
    t["up"] = dev_bf16(inputs.activations(g, 8, k), gpu)
    out = {
        "q8": _u8(bq.q8_1_act_bytes(m, k), gpu),
        "mmq": empty_bf16((m, n), gpu),
        "gemv1": empty_bf16((n,), gpu),
        "gemv2": empty_bf16((2, n), gpu),
        "gemv4": empty_bf16((4, n), gpu),
        "gemv8": empty_bf16((8, n), gpu),
        "fused8": empty_bf16((8, n), gpu),
        "silu": empty_bf16((8, k), gpu),
        "q8h": _u8(bq.q8_1_act_bytes(8, k), gpu),
        "deq": empty_bf16((n, k), gpu),
        "dense": empty_bf16((m, n), gpu),
        "prefill": empty_bf16((m, n), gpu),
        "mmq4": empty_bf16((m, n4), gpu),
        "gemv4k": empty_bf16((n4,), gpu),
        "wq4k": _u8(bq.q4k_weight_bytes(n4, k), gpu),
    }
    return (m, n, k, n4), t, out


def _run(dims, t, o):
    m, n, k, n4 = dims
    act = t["act"]
    bq.quantize_act_q8_1(act, o["q8"], m, k)
    bq.q2_0_mmq_gemm(o["q8"], t["w2"], o["mmq"], m, n, k)
    bq.q2_0_gemv_vec(act[0], t["w2"], o["gemv1"], n, k)
    bq.q2_0_gemv_vec_batchm(act[:2], t["w2"], o["gemv2"], 2, n, k)
    bq.q2_0_gemv_vec_batchm(act[:4], t["w2"], o["gemv4"], 4, n, k)
    bq.q2_0_gemv_vec_batchm(act[:8], t["w2"], o["gemv8"], 8, n, k)
    bq.q2_0_gemv_gate_up_silu(act[:8], t["w2"], t["w2"], o["fused8"], 8, n, k)
    bq.silu_mul_bf16(t["gate"], t["up"], o["silu"])
    bq.silu_mul_quantize_q8_1(t["gate"], t["up"], o["q8h"], 8, k)
    bq.dequant_q2_0_to_bf16(t["w2"], o["deq"], n, k)
    bq.dense_gemm_bf16(act, o["deq"], o["dense"], m, n, k)
    bq.q2_0_prefill_gemm_noalloc(act, t["w2"], o["prefill"], m, n, k)
    bq.q4k_mmq_gemm(o["q8"], t["w4"], o["mmq4"], m, n4, k)
    bq.q4k_gemv_vec(act[0], t["w4"], o["gemv4k"], n4, k)
    bq.quantize_weight_q4k(t["wbf"], o["wq4k"], n4, k)


def test_graph_replays_match_eager(gpu):
    dims, t, o = _setup(gpu)
    _run(dims, t, o)
    torch.cuda.synchronize()
    eager = {key: v.clone() for key, v in o.items()}
    # the eager results are real: nonzero, and the chained ones differ from their inputs
    for key in ("mmq", "gemv1", "fused8", "dense", "mmq4", "gemv4k"):
        assert torch.count_nonzero(eager[key].view(torch.int16)) > 0, key

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _run(dims, t, o)  # warm the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        _run(dims, t, o)
    torch.cuda.synchronize()

    busy_a = torch.randn((512, 512), device=gpu)
    for rep in range(3):
        for v in o.values():
            v.zero_()
        busy_b = busy_a @ busy_a  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(busy_b).all()
        for key, v in o.items():
            a = v.view(torch.uint8) if v.dtype != torch.uint8 else v
            b = eager[key].view(torch.uint8) if eager[key].dtype != torch.uint8 else eager[key]
            assert torch.equal(a, b), f"replay {rep}: {key} differs from the eager result"


def test_concurrent_streams_match_eager(gpu):
    # Two streams (default priority) run disjoint halves of the calls at the
    # same time; no entry point but the no-allocation one keeps state between
    # calls, so each output equals the eager result bit for bit.
    dims, t, o = _setup(gpu)
    _run(dims, t, o)
    torch.cuda.synchronize()
    eager = {key: v.clone() for key, v in o.items()}
    for v in o.values():
        v.zero_()
    torch.cuda.synchronize()
    m, n, k, n4 = dims
    act = t["act"]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(s1):
            bq.quantize_act_q8_1(act, o["q8"], m, k)
            bq.q2_0_mmq_gemm(o["q8"], t["w2"], o["mmq"], m, n, k)
            bq.q4k_mmq_gemm(o["q8"], t["w4"], o["mmq4"], m, n4, k)
            bq.dequant_q2_0_to_bf16(t["w2"], o["deq"], n, k)
            bq.dense_gemm_bf16(act, o["deq"], o["dense"], m, n, k)
        with torch.cuda.stream(s2):
            bq.q2_0_gemv_vec(act[0], t["w2"], o["gemv1"], n, k)
            bq.q2_0_gemv_vec_batchm(act[:2], t["w2"], o["gemv2"], 2, n, k)
            bq.q2_0_gemv_vec_batchm(act[:4], t["w2"], o["gemv4"], 4, n, k)
            bq.q2_0_gemv_vec_batchm(act[:8], t["w2"], o["gemv8"], 8, n, k)
            bq.q2_0_gemv_gate_up_silu(act[:8], t["w2"], t["w2"], o["fused8"], 8, n, k)
            bq.silu_mul_bf16(t["gate"], t["up"], o["silu"])
            bq.silu_mul_quantize_q8_1(t["gate"], t["up"], o["q8h"], 8, k)
            bq.q4k_gemv_vec(act[0], t["w4"], o["gemv4k"], n4, k)
            bq.quantize_weight_q4k(t["wbf"], o["wq4k"], n4, k)
    torch.cuda.synchronize()
    for key, v in o.items():
        if key == "prefill":
            continue  # the no-allocation entry point is not run here
        a = v.view(torch.uint8) if v.dtype != torch.uint8 else v
        b = eager[key].view(torch.uint8) if eager[key].dtype != torch.uint8 else eager[key]
        assert torch.equal(a, b), f"{key} differs from the eager result"


def test_graph_replays_balanced_gemv(gpu):
    # The batched GEMV's balanced launch (one workgroup of ceil(n / units) rows
    # per compute unit, its LDS attribute set on first use), single and fused,
    # captured after an eager run and replayed three times.
    g = inputs.rng(93)
    m, n, k = 8, 12288 + 1, 1024
    x = dev_bf16(inputs.activations(g, m, k, outliers=True), gpu)
    wg, wu = dev_u8(inputs.q2_0_weight(g, n, k), gpu), dev_u8(inputs.q2_0_weight(g, n, k), gpu)
    single, fused = empty_bf16((m, n), gpu), empty_bf16((m, n), gpu)

    def run():
        bq.q2_0_gemv_vec_batchm(x, wg, single, m, n, k)
        bq.q2_0_gemv_gate_up_silu(x, wg, wu, fused, m, n, k)

    run()
    torch.cuda.synchronize()
    eager = (single.clone(), fused.clone())
    assert torch.count_nonzero(eager[0].view(torch.int16)) > 0
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        single.zero_()
        fused.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(single.view(torch.int16), eager[0].view(torch.int16)), f"replay {rep}: single"
        assert torch.equal(fused.view(torch.int16), eager[1].view(torch.int16)), f"replay {rep}: fused"

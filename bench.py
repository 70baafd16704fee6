"""Benchmark of the packed low-bit weight-quantized matmul hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one pass of the whole hot path over one batch of synthetic
input, every leg on the current stream, each leg captured once into a HIP
graph and replayed between HIP events:
  decode   : 1000 x q2_0_gemv_vec, qkvz n=12288 k=2048 (m=1), the weight
             rotated through 80 copies (537 MB > the 256 MB Infinity Cache) so
             that every call streams its weight from HBM; and the same calls
             on one copy (warm, served from the Infinity Cache);
  verify   : q2_0_gemv_vec_batchm chain gate -> up -> silu_mul -> down,
             FFN [17408, 5120] / [5120, 17408], m in {2, 3, 4, 8}; and the same
             step with q2_0_gemv_gate_up_silu in place of the first three calls;
             both rotated through 8 copies of the three weights (568 MB);
  prefill  : quantize_act_q8_1 and q2_0_mmq_gemm, qkvz n=12288 k=2048, m in
             {512, 2048}, apart and end to end; and the bf16 fallback
             (dequant + dense GEMM) at both m;
  ffn      : m=4096 FFN prefill, Q2_0 and Q4_K: quantize, gate and up MMQ
             (sharing the quantized input), silu_mul fused into the down
             projection's quantization, down MMQ; each format against the
             peak of the MFMA it contracts on (int8 for Q2_0, fp16 for Q4_K);
  q4k      : Q4_K decode GEMV (m=1) on the FFN gate [17408, 5120] and down
             [5120, 17408] shapes, each weight rotated through 8 copies
             (401 MB); and the Q4_K weight quantizer on a bf16 [17408, 5120]
             weight (two input/output pairs alternate);
  ceilings : what the GPU reaches on each path alone (ceilings/ceilings.hip,
             a library of its own): an empty kernel (the launch floor, one
             workgroup and the decode GEMV's grid), a cold streaming read of
             the decode GEMV's 6,713,344 bytes per launch with its grid
             (rotated through 80 buffers), back-to-back int8 and fp16 MFMAs
             (the Q2_0 and the Q4_K MMQ's instructions), back-to-back 24-bit
             integer multiply-adds on the vector ALU, the MFMA loops with the
             MMQs' numbers of VALU instructions per MFMA interleaved, and LDS
             read and write bandwidth;
  copy     : (not in the default set) a plain 256 MiB device-to-device copy,
             the known-size reference for the HBM byte counters.
The JSON line reports the decode GEMV (the workload the headline metric is
quoted on) as `value`, with its roofline (against the published peak and
against the measured streaming ceiling) and the CPU oracle beside it; the
m = 2048 MMQ under "prefill" the same way; every other leg under "legs" and
the oracle's figures for the other workloads under "cpu_baselines".  Inputs
are resident in HBM before the timed region starts.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Q2_0 MMQ prefill int8 TOPS + GEMV decode HBM GB/s (% of MI355X peak)"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
INT8_PEAK_TOPS = 5033.0      # MI355X dense int8 MFMA, published (no sparsity)
BF16_PEAK_TFLOPS = 2516.0    # MI355X dense bf16 MFMA, published
FP16_PEAK_TFLOPS = 2516.0    # MI355X dense fp16 MFMA, published (the Q4_K MMQ contracts in fp16)
VALU_PEAK_GINSTR = 256 * 4 * 2.4e9 / 4 / 1e9  # wave64 VALU instructions/s: 4 SIMDs/CU, 4 cycles each

DECODE_CALLS = 1000
DECODE_COPIES = 80
VERIFY_COPIES = 8
COPY_BYTES = 256 << 20
DECODE_BYTES = 12288 * 2048 * 17 // 64 + 2 * 2048 + 2 * 12288  # 6,713,344
# Per-dispatch HBM traffic of the decode GEMV and of the m = 2048 MMQ, measured
# with rocprofv3 counters (FETCH_SIZE + WRITE_SIZE, scaled by the same counters
# on the copy leg).  A figure is reported only while the kernel source still
# matches the hash the counters were taken with.
_CSRC = os.path.join(ROOT, "bit_quantized_matmul_quantize_amd", "csrc")
TRAFFIC_DECODE = (os.path.join(ROOT, "profiles", "hbm_traffic_decode_gemv_n12288_k2048.txt"),
                  os.path.join(_CSRC, "gemv.hip"))
TRAFFIC_MMQ = (os.path.join(ROOT, "profiles", "hbm_traffic_q2_0_mmq_m2048_n12288_k2048.txt"),
               os.path.join(_CSRC, "mmq_q2.hip"))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=24.0,
                   help="target CPU time of all the oracle samples together")
    p.add_argument("--legs", default="decode,verify,prefill,ffn,q4k,ceilings")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Leg:
    """A captured HIP graph plus its event timings.

    `keep` holds every tensor the captured kernels touch: the graph stores raw
    device pointers, and torch.cuda.graph() empties the allocator cache when a
    later capture begins, so a tensor without a live reference would be
    unmapped under an earlier graph."""

    def __init__(self, name, fn, keep, launches, work, unit, kernel, peak, bound, min_ms=2.0, peak_unit=None):
        import torch
        self.name, self.fn, self.keep = name, fn, list(keep)
        self.unit, self.kernel, self.peak, self.bound = unit, kernel, peak, bound
        log(f"capture {name}")
        fn()  # eager run first: argument errors surface here, outside capture
        torch.cuda.synchronize()
        # Repeat the leg inside one graph until a replay lasts >= min_ms, so the
        # fixed cost of launching a graph is amortized over many kernels.
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        self.reps = max(1, min(200, int(np.ceil(min_ms / max(a.elapsed_time(b), 1e-3)))))
        self.launches = launches * self.reps
        self.work = work * self.reps
        self.graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(self.graph):
            for _ in range(self.reps):
                fn()
        torch.cuda.synchronize()
        self.ms = []

    def run(self, timed):
        import torch
        if timed:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            self.graph.replay()
            b.record()
            self._pending = (a, b)
        else:
            self.graph.replay()

    def collect(self):
        a, b = self._pending
        self.ms.append(a.elapsed_time(b))

    def summary(self):
        ms = float(np.mean(self.ms))
        per_launch_us = ms * 1e3 / self.launches
        rate = self.work / (ms * 1e-3)  # units per second
        scale = {"GB/s": 1e9, "TOPS": 1e12, "Ginstr/s": 1e9, "launches/s": 1.0}[self.unit]
        achieved = rate / scale
        out = dict(name=self.name, ms=round(ms, 4), reps=self.reps, us_per_launch=round(per_launch_us, 3),
                   value=round(achieved, 2), unit=self.unit, kernel=self.kernel, bound=self.bound)
        if self.peak:
            out["frac_of_peak"] = round(achieved / self.peak, 4)
        return out


class Rotation:
    """Cycles through weight copies, one per call at capture time, so a graph
    of many calls reads every copy in turn."""

    def __init__(self, copies):
        self.copies, self.i = copies, 0

    def next(self):
        c = self.copies[self.i % len(self.copies)]
        self.i += 1
        return c


def decode_legs(bq, dev, d):
    """1000 m=1 GEMV calls: weight rotated through DECODE_COPIES copies (cold)
    and on one copy (warm)."""
    import torch
    n, k = d["n"], d["k"]
    w0 = torch.from_numpy(d["w"]).to(dev)
    wcopies = [w0] + [w0.clone() for _ in range(DECODE_COPIES - 1)]
    x = torch.from_numpy(d["act"][0].copy().view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.empty((n,), dtype=torch.bfloat16, device=dev)

    def cold():
        for i in range(DECODE_CALLS):
            bq.q2_0_gemv_vec(x, wcopies[i % DECODE_COPIES], y, n, k)

    def warm():
        for _ in range(DECODE_CALLS):
            bq.q2_0_gemv_vec(x, w0, y, n, k)

    bytes_per_call = w0.numel() + 2 * k + 2 * n
    assert bytes_per_call == DECODE_BYTES
    return [Leg("decode_gemv_m1", cold, wcopies + [x, y], DECODE_CALLS, DECODE_CALLS * bytes_per_call, "GB/s",
                "q2_0_gemv1_kernel", HBM_PEAK_GBS, "hbm"),
            Leg("decode_gemv_m1_warm", warm, [w0, x, y], DECODE_CALLS, DECODE_CALLS * bytes_per_call, "GB/s",
                "q2_0_gemv1_kernel (one weight copy, Infinity Cache)", HBM_PEAK_GBS, "hbm")]


def verify_leg(bq, dev, Wcopies, act, m, H, I):
    import torch
    x = torch.from_numpy(np.ascontiguousarray(act[:m]).view(np.int16)).to(dev).view(torch.bfloat16)
    g_ = torch.empty((m, I), dtype=torch.bfloat16, device=dev)
    u_ = torch.empty((m, I), dtype=torch.bfloat16, device=dev)
    o_ = torch.empty((m, H), dtype=torch.bfloat16, device=dev)
    rot = Rotation(Wcopies)

    def fn():
        wg, wu, wd = rot.next()
        bq.q2_0_gemv_vec_batchm(x, wg, g_, m, I, H)
        bq.q2_0_gemv_vec_batchm(x, wu, u_, m, I, H)
        bq.silu_mul_bf16(g_, u_, g_, m * I)
        bq.q2_0_gemv_vec_batchm(g_, wd, o_, m, H, I)

    wg, wu, wd = Wcopies[0]
    work = wg.numel() + wu.numel() + wd.numel() + m * (6 * H + 12 * I)
    kname = (f"q2_0_gemv_mfma_kernel<{m}> x3 + silu_mul" if m >= 3 else
             f"q2_0_gemvp_kernel<{m}> gate, up + silu_mul + q2_0_gemvm_kernel<{m}> down")
    keep = [t for c in Wcopies for t in c] + [x, g_, u_, o_]
    return Leg(f"verify_ffn_m{m}", fn, keep, 4, work, "GB/s", kname, HBM_PEAK_GBS, "hbm")


def verify_fused_leg(bq, dev, Wcopies, act, m, H, I):
    """The same FFN step with gate, up and silu_mul fused into one launch."""
    import torch
    x = torch.from_numpy(np.ascontiguousarray(act[:m]).view(np.int16)).to(dev).view(torch.bfloat16)
    h_ = torch.empty((m, I), dtype=torch.bfloat16, device=dev)
    o_ = torch.empty((m, H), dtype=torch.bfloat16, device=dev)
    rot = Rotation(Wcopies)

    def fn():
        wg, wu, wd = rot.next()
        bq.q2_0_gemv_gate_up_silu(x, wg, wu, h_, m, I, H)
        bq.q2_0_gemv_vec_batchm(h_, wd, o_, m, H, I)

    wg, wu, wd = Wcopies[0]
    work = wg.numel() + wu.numel() + wd.numel() + m * (2 * H + 4 * I)
    kname = (f"q2_0_gemv_mfma_kernel<{m}> gate+up+silu, q2_0_gemv_mfma_kernel<{m}> down" if m >= 3 else
             f"q2_0_gemvp_kernel<{m}> gate+up+silu, q2_0_gemvm_kernel<{m}> down")
    keep = [t for c in Wcopies for t in c] + [x, h_, o_]
    return Leg(f"verify_ffn_fused_m{m}", fn, keep, 2, work, "GB/s", kname, HBM_PEAK_GBS, "hbm")


def copy_leg(dev):
    """Known-size reference for the byte counters: one 256 MiB device copy."""
    import torch
    src = torch.randint(0, 255, (COPY_BYTES,), dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    return Leg("copy_256MiB", lambda: dst.copy_(src), [src, dst], 1, 2 * COPY_BYTES, "GB/s",
               "device copy", HBM_PEAK_GBS, "hbm")


def measured_traffic(summary):
    """Bytes per dispatch from a committed counter summary (path, kernel
    source), or None when it is missing or was taken on another version of
    the kernel."""
    import hashlib
    path, source = summary
    try:
        fields = dict(line.split(":", 1) for line in open(path) if ":" in line)
        digest = hashlib.sha256(open(source, "rb").read()).hexdigest()
        if fields.get("kernel_source_sha256", "").strip() != digest:
            return None
        return int(fields["traffic_bytes_per_launch"].strip())
    except (OSError, KeyError, ValueError):
        return None


def prefill_legs(bq, dev, p):
    import torch
    n, k = p["n"], p["k"]
    w = torch.from_numpy(p["w"]).to(dev)
    scratch = torch.empty((n * k,), dtype=torch.bfloat16, device=dev)
    bq.dequant_q2_0_to_bf16(w, scratch, n, k, 128)  # the dense GEMM legs read the dequantized weight
    legs = []
    for m in (512, 2048):
        x = torch.from_numpy(np.ascontiguousarray(p["act"][:m]).view(np.int16)).to(dev).view(torch.bfloat16)
        q8 = torch.empty((bq.q8_1_act_bytes(m, k),), dtype=torch.uint8, device=dev)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        bq.quantize_act_q8_1(x, q8, m, k)
        keep = [w, x, q8, y]
        legs.append(Leg(f"prefill_mmq_m{m}", lambda m=m, q8=q8, y=y: bq.q2_0_mmq_gemm(q8, w, y, m, n, k),
                        keep, 1, 2.0 * m * n * k, "TOPS", "q2_0_mmq_kernel", INT8_PEAK_TOPS, "mfma"))
        legs.append(Leg(f"prefill_quantize_m{m}", lambda m=m, x=x, q8=q8: bq.quantize_act_q8_1(x, q8, m, k),
                        keep, 1, 2 * m * k + bq.q8_1_act_bytes(m, k), "GB/s", "quantize_q8_1_kernel",
                        HBM_PEAK_GBS, "hbm"))
        legs.append(Leg(f"prefill_quantize_mmq_m{m}",
                        lambda m=m, x=x, q8=q8, y=y: bq.q2_0_prefill_gemm(x, w, y, None, q8, m, n, k, 128, True),
                        keep, 2, 2.0 * m * n * k, "TOPS", "quantize_q8_1_kernel + q2_0_mmq_kernel",
                        INT8_PEAK_TOPS, "mfma"))
        legs.append(Leg(f"fallback_dense_gemm_m{m}", lambda m=m, x=x, y=y: bq.dense_gemm_bf16(x, scratch, y, m, n, k),
                        [x, scratch, y], 1, 2.0 * m * n * k, "TOPS", "dense_gemm_bf16_kernel", BF16_PEAK_TFLOPS,
                        "mfma"))
    legs.append(Leg("fallback_dequant", lambda: bq.dequant_q2_0_to_bf16(w, scratch, n, k, 128), [w, scratch],
                    1, w.numel() + 2 * n * k, "GB/s", "dequant_q2_0_kernel", HBM_PEAK_GBS, "hbm"))
    return legs


def ffn_legs(bq, dev, F):
    import torch
    H, I, m = F["hidden"], F["inter"], 4096
    x = torch.from_numpy(np.ascontiguousarray(F["act"]).view(np.int16)).to(dev).view(torch.bfloat16)
    q8a = torch.empty((bq.q8_1_act_bytes(m, H),), dtype=torch.uint8, device=dev)
    q8h = torch.empty((bq.q8_1_act_bytes(m, I),), dtype=torch.uint8, device=dev)
    gate = torch.empty((m, I), dtype=torch.bfloat16, device=dev)
    up = torch.empty((m, I), dtype=torch.bfloat16, device=dev)
    out = torch.empty((m, H), dtype=torch.bfloat16, device=dev)
    legs = []
    # each format against the peak of the MFMA type its contraction runs on
    for fmt, key, gemm, kname, peak in (("q2_0", "q2", bq.q2_0_mmq_gemm, "q2_0_mmq_kernel", INT8_PEAK_TOPS),
                                        ("q4k", "q4k", bq.q4k_mmq_gemm, "q4k_mmq_kernel", FP16_PEAK_TFLOPS)):
        wg, wu, wd = (torch.from_numpy(F[key][name]).to(dev) for name in ("wg", "wu", "wd"))

        def ffn(wg=wg, wu=wu, wd=wd, gemm=gemm):
            bq.quantize_act_q8_1(x, q8a, m, H)
            gemm(q8a, wg, gate, m, I, H)
            gemm(q8a, wu, up, m, I, H)
            bq.silu_mul_quantize_q8_1(gate, up, q8h, m, I)
            gemm(q8h, wd, out, m, H, I)

        keep = [wg, wu, wd, x, q8a, q8h, gate, up, out]
        legs.append(Leg(f"ffn_prefill_{fmt}_m4096", ffn, keep, 5, 3 * 2.0 * m * H * I, "TOPS",
                        f"{kname} x3 + quantize + silu_mul_quantize", peak, "mfma"))
        legs.append(Leg(f"ffn_gate_proj_{fmt}_m4096", lambda wg=wg, gemm=gemm: gemm(q8a, wg, gate, m, I, H),
                        keep, 1, 2.0 * m * H * I, "TOPS", kname, peak, "mfma"))
        legs.append(Leg(f"ffn_down_proj_{fmt}_m4096", lambda wd=wd, gemm=gemm: gemm(q8h, wd, out, m, H, I),
                        keep, 1, 2.0 * m * H * I, "TOPS", kname, peak, "mfma"))
    return legs


def q4k_legs(bq, dev, Q):
    import torch
    legs = []
    copies, calls = 8, 64
    for name, wkey, akey, n, k in (("q4k_decode_gate", "w_gate", "a_gate", Q["inter"], Q["hidden"]),
                                   ("q4k_decode_down", "w_down", "a_down", Q["hidden"], Q["inter"])):
        w0 = torch.from_numpy(Q[wkey]).to(dev)
        ws = [w0] + [w0.clone() for _ in range(copies - 1)]
        x = torch.from_numpy(Q[akey][0].copy().view(np.int16)).to(dev).view(torch.bfloat16)
        y = torch.empty((n,), dtype=torch.bfloat16, device=dev)

        def fn(ws=ws, x=x, y=y, n=n, k=k):
            for i in range(calls):
                bq.q4k_gemv_vec(x, ws[i % copies], y, n, k)

        legs.append(Leg(f"{name}_n{n}_k{k}", fn, ws + [x, y], calls, calls * (w0.numel() + 2 * k + 2 * n),
                        "GB/s", "q4k_gemv1_kernel", HBM_PEAK_GBS, "hbm"))
    n, k = Q["inter"], Q["hidden"]
    xb = [torch.from_numpy(Q["w_bf16"].view(np.int16)).to(dev).view(torch.bfloat16)]
    xb.append(xb[0].clone())
    qs = [torch.empty((bq.q4k_weight_bytes(n, k),), dtype=torch.uint8, device=dev) for _ in range(2)]

    def quant():
        for i in range(2):
            bq.quantize_weight_q4k(xb[i], qs[i], n, k)

    legs.append(Leg(f"q4k_quantize_weight_n{n}_k{k}", quant, xb + qs, 2, 2 * (2 * n * k + qs[0].numel()),
                    "GB/s", "quantize_weight_q4k_kernel", HBM_PEAK_GBS, "hbm"))
    return legs


def ceiling_legs(dev, gemv_blocks):
    """Measured ceilings (ceilings/ceilings.hip): launch floor, cold streaming
    read of the decode GEMV's bytes with its grid, int8 and fp16 MFMA and
    VALU issue rates, MFMA rates at the MMQs' VALU mixes, LDS bandwidth."""
    import torch
    import ceilings

    stream = lambda: ctypes_stream(torch)
    legs = []
    calls = 1000
    for label, blocks, threads in (("1x64", 1, 64), (f"{gemv_blocks}x256", gemv_blocks, 256)):
        legs.append(Leg(f"ceiling_empty_kernel_{label}",
                        lambda b=blocks, t=threads: [ceilings.call("ceil_empty", b, t, stream())
                                                     for _ in range(calls)],
                        [], calls, calls, "launches/s", "empty_kernel", None, "launch"))
    bufs = [torch.empty((DECODE_BYTES,), dtype=torch.uint8, device=dev).random_(0, 255)
            for _ in range(DECODE_COPIES)]
    sink = torch.zeros((max(gemv_blocks, 4096),), dtype=torch.int32, device=dev)
    legs.append(Leg("ceiling_stream_read_6713344B",
                    lambda: [ceilings.call("ceil_stream_read", bufs[i % DECODE_COPIES].data_ptr(), DECODE_BYTES,
                                           sink.data_ptr(), gemv_blocks, stream()) for i in range(calls)],
                    bufs + [sink], calls, calls * DECODE_BYTES, "GB/s", "stream_read_kernel (cold, 80 buffers)",
                    HBM_PEAK_GBS, "hbm"))
    out = torch.empty((12288,), dtype=torch.bfloat16, device=dev)
    legs.append(Leg("ceiling_stream_read_write_6713344B",
                    lambda: [ceilings.call("ceil_stream_read_write", bufs[i % DECODE_COPIES].data_ptr(),
                                           DECODE_BYTES - 2 * 12288, out.data_ptr(), 12288, gemv_blocks, stream())
                             for i in range(calls)],
                    bufs + [out], calls, calls * DECODE_BYTES, "GB/s",
                    "stream_read_write_kernel (cold, 80 buffers; 24 KB written)", HBM_PEAK_GBS, "hbm"))
    iters = 4096
    for blocks in (512, 1024):
        ops = blocks * 4 * iters * 4 * 2.0 * 32 * 32 * 32
        legs.append(Leg(f"ceiling_mfma_i8_{blocks}x256",
                        lambda b=blocks: ceilings.call("ceil_mfma_i8", b, iters, sink.data_ptr(), stream()),
                        [sink], 1, ops, "TOPS", "v_mfma_i32_32x32x32_i8 loop", INT8_PEAK_TOPS, "mfma"))
    for blocks in (512, 1024):
        ops = blocks * 4 * iters * 4 * 2.0 * 32 * 32 * 16
        legs.append(Leg(f"ceiling_mfma_f16_{blocks}x256",
                        lambda b=blocks: ceilings.call("ceil_mfma_f16", b, iters, sink.data_ptr(), stream()),
                        [sink], 1, ops, "TOPS", "v_mfma_f32_32x32x16_f16 loop", FP16_PEAK_TFLOPS, "mfma"))
    viters = 8192
    for blocks in (1024, 2048):
        instr = blocks * 4 * viters * 8
        legs.append(Leg(f"ceiling_valu_mad_i24_{blocks}x256",
                        lambda b=blocks: ceilings.call("ceil_valu_mad", b, viters, sink.data_ptr(), stream()),
                        [sink], 1, instr, "Ginstr/s", "v_mad_i32_i24 loop", VALU_PEAK_GINSTR, "valu"))
    # the MMQs' instruction mixes: four MFMAs and 4v multiply-adds per iteration
    # (v = 24: the Q2_0 fold's VALU per int8 MFMA; 33: that kernel's whole mix;
    # 14: the Q4_K kernel's per fp16 MFMA), two waves per SIMD as in the kernels
    miters = 1024
    for f16, per4, label in ((0, 96, "i8_24valu"), (0, 132, "i8_33valu"), (1, 56, "f16_14valu")):
        ops = 512 * 4 * miters * 4 * 2.0 * 32 * 32 * (16 if f16 else 32)
        legs.append(Leg(f"ceiling_mix_{label}_512x256",
                        lambda f=f16, v=per4: ceilings.call("ceil_mix", 512, miters, f, v, sink.data_ptr(), stream()),
                        [sink], 1, ops, "TOPS",
                        f"{'v_mfma_f32_32x32x16_f16' if f16 else 'v_mfma_i32_32x32x32_i8'} + {per4 // 4} "
                        f"v_mad_i32_i24 per MFMA", FP16_PEAK_TFLOPS if f16 else INT8_PEAK_TOPS, "mfma"))
    # LDS bandwidth, 16-byte accesses by every lane, two workgroups per CU
    liters = 2048
    for write in (0, 1):
        nbytes = 512 * 256 * liters * 16 * 16
        legs.append(Leg(f"ceiling_lds_{'write' if write else 'read'}_b128",
                        lambda w=write: ceilings.call("ceil_lds", 512, liters, w, sink.data_ptr(), stream()),
                        [sink], 1, nbytes, "GB/s", f"ds_{'write' if write else 'read'}_b128 loop", None, "lds"))
    return legs


def ctypes_stream(torch):
    return torch.cuda.current_stream().cuda_stream


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def timed_oracle(fn, budget_s, max_calls):
    """Calls fn until budget_s of CPU time or max_calls; returns (calls, seconds)."""
    calls, t = 0, 0.0
    while (t < budget_s and calls < max_calls) or calls == 0:
        t1 = time.perf_counter()
        fn()
        t += time.perf_counter() - t1
        calls += 1
    return calls, t


def cpu_baselines(ctx, budget):
    """The oracle on one pinned host core, on bounded samples of each workload:
    the tiny case whole, the decode GEMV in whole calls, the m = 2 verify chain
    whole, the m = 2048 prefill MMQ and the m = 4096 FFN chains (Q2_0 and
    Q4_K) on 16 activation rows with all n (their cost is linear in rows),
    extrapolated."""
    import oracle
    import inputs
    try:
        os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
    except Exception:
        pass
    host = f"one pinned core of {os.cpu_count()}, {cpu_model()}"
    out = {}
    if "tiny" in ctx:
        d = ctx["tiny"]
        m, n, k = d["m"], d["n"], d["k"]

        def c1():
            q8, _ = oracle.quantize_act_q8_1(d["act"], m, k)
            oracle.q2_0_mmq(q8, d["w"], m, n, k)
            oracle.q2_0_gemv(d["act"][:1], d["w"], 1, n, k)

        calls, t = timed_oracle(c1, 0.05 * budget, 2000)
        out["tiny_m4_n256_k512"] = {"value": round(2.0 * m * n * k * calls / t / 1e12, 6), "unit": "TOPS", "cores": 1,
                          "kind": "oracle", "ms_per_call": round(t * 1e3 / calls, 3),
                          "sample": f"{calls} whole tiny passes (quantize, MMQ m=4 n=256 k=512, GEMV row 0), "
                                    f"{t:.2f} s on {host}; TOPS counts the MMQ's 2mnk"}
    if "decode" in ctx:
        d = ctx["decode"]
        calls, t = timed_oracle(lambda: oracle.q2_0_gemv(d["act"], d["w"], 1, d["n"], d["k"]), 0.4 * budget, 200)
        out["decode_gemv_n12288_k2048"] = {"value": round(calls * DECODE_BYTES / t / 1e9, 4), "unit": "GB/s", "cores": 1,
                            "kind": "oracle",
                            "sample": f"{calls} decode GEMV calls (n=12288, k=2048) of the oracle, {t:.1f} s on {host}"}
    if "verify" in ctx:
        f, m = ctx["verify"], 2
        H, I = f["hidden"], f["inter"]
        calls, t = timed_oracle(lambda: oracle.ffn_chain_gemv(np.ascontiguousarray(f["act"][:m]), f["wg"], f["wu"],
                                                              f["wd"], m, H, I), 0.15 * budget, 20)
        work = f["wg"].size + f["wu"].size + f["wd"].size + m * (6 * H + 12 * I)
        out["verify_ffn_m2"] = {"value": round(calls * work / t / 1e9, 4), "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{calls} whole m=2 verify chains (gate, up, silu_mul, down; 71 MB of "
                                         f"weights), {t:.1f} s on {host}"}
    if "prefill" in ctx:
        p, rows = ctx["prefill"], 16
        n, k = p["n"], p["k"]
        q8_rows, _ = oracle.quantize_act_q8_1(np.ascontiguousarray(p["act"][:rows]), rows, k)
        calls, t = timed_oracle(lambda: oracle.q2_0_mmq(q8_rows, p["w"], rows, n, k), 0.1 * budget, 50)
        out["prefill_qkvz_mmq_m2048"] = {
            "value": round(2.0 * rows * n * k * calls / t / 1e12, 6), "unit": "TOPS", "cores": 1, "kind": "oracle",
            "extrapolated_ms_m2048": round(t * 1e3 / calls * 2048 / rows, 1),
            "sample": f"{calls} oracle MMQ calls on {rows} of the 2048 activation rows (n=12288, k=2048), "
                      f"{t:.1f} s on {host}; extrapolated from 16 rows (the oracle's cost is linear in rows)"}
    if "ffn" in ctx:
        F, rows = ctx["ffn"], 16
        H, I = F["hidden"], F["inter"]
        x = np.ascontiguousarray(F["act"][:rows])
        W = F["q2"]

        def c5():
            q8, _ = oracle.quantize_act_q8_1(x, rows, H)
            g = oracle.round_bf16(oracle.q2_0_mmq(q8, W["wg"], rows, I, H))
            u = oracle.round_bf16(oracle.q2_0_mmq(q8, W["wu"], rows, I, H))
            q8h, _ = oracle.quantize_act_q8_1(oracle.silu_mul_bf16(g, u), rows, I)
            oracle.q2_0_mmq(q8h, W["wd"], rows, H, I)

        calls, t = timed_oracle(c5, 0.15 * budget, 5)
        out["ffn_prefill_q2_0_m4096"] = {
            "value": round(3 * 2.0 * rows * H * I * calls / t / 1e12, 6), "unit": "TOPS", "cores": 1,
            "kind": "oracle", "extrapolated_ms_m4096": round(t * 1e3 / calls * 4096 / rows, 1),
            "sample": f"{calls} oracle Q2_0 FFN chains (quantize, gate, up, silu_mul, quantize, down) on {rows} of "
                      f"the 4096 rows, {t:.1f} s on {host}; extrapolated from 16 rows (linear in rows)"}
        if "q4k" in F:
            W4 = F["q4k"]

            def c5k():
                q8, _ = oracle.quantize_act_q8_1(x, rows, H)
                g = oracle.round_bf16(oracle.q4k_mmq(q8, W4["wg"], rows, I, H))
                u = oracle.round_bf16(oracle.q4k_mmq(q8, W4["wu"], rows, I, H))
                q8h, _ = oracle.quantize_act_q8_1(oracle.silu_mul_bf16(g, u), rows, I)
                oracle.q4k_mmq(q8h, W4["wd"], rows, H, I)

            calls, t = timed_oracle(c5k, 0.15 * budget, 5)
            out["ffn_prefill_q4k_m4096"] = {
                "value": round(3 * 2.0 * rows * H * I * calls / t / 1e12, 6), "unit": "TOPS", "cores": 1,
                "kind": "oracle", "extrapolated_ms_m4096": round(t * 1e3 / calls * 4096 / rows, 1),
                "sample": f"{calls} oracle Q4_K FFN chains (quantize, gate, up, silu_mul, quantize, down) on {rows} "
                          f"of the 4096 rows, {t:.1f} s on {host}; extrapolated from 16 rows (linear in rows)"}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU: the path has no inter-GPU "
                          "sharding (--gpus must be 1)", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import bit_quantized_matmul_quantize_amd as bq
    import inputs

    dev = torch.device("cuda:0")
    legs_wanted = set(args.legs.split(","))
    legs = []
    ctx = {"tiny": inputs.tiny()}
    if "decode" in legs_wanted:
        ctx["decode"] = inputs.decode_gemv()
        legs += decode_legs(bq, dev, ctx["decode"])
    if "verify" in legs_wanted:
        f = ctx["verify"] = inputs.verify_ffn()
        W0 = tuple(torch.from_numpy(f[key]).to(dev) for key in ("wg", "wu", "wd"))
        Wcopies = [W0] + [tuple(t.clone() for t in W0) for _ in range(VERIFY_COPIES - 1)]
        for m in (2, 3, 4, 8):
            legs.append(verify_leg(bq, dev, Wcopies, f["act"], m, f["hidden"], f["inter"]))
        for m in (2, 3, 4, 8):
            legs.append(verify_fused_leg(bq, dev, Wcopies, f["act"], m, f["hidden"], f["inter"]))
    if "prefill" in legs_wanted:
        ctx["prefill"] = inputs.prefill_qkvz()
        legs += prefill_legs(bq, dev, ctx["prefill"])
    if "ffn" in legs_wanted:
        ctx["ffn"] = inputs.prefill_ffn()
        legs += ffn_legs(bq, dev, ctx["ffn"])
    if "q4k" in legs_wanted:
        legs += q4k_legs(bq, dev, inputs.q4k_decode())
    if "ceilings" in legs_wanted:
        legs += ceiling_legs(dev, gemv_blocks=12288 // 24)  # the decode GEMV's grid: 24 rows per workgroup
    if "copy" in legs_wanted:
        legs.append(copy_leg(dev))

    # ---- timed region ----------------------------------------------------------
    log(f"{len(legs)} legs captured; warmup {args.warmup}, steps {args.steps}")
    for _ in range(args.warmup):
        for leg in legs:
            leg.run(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for step in range(args.steps):
        for leg in legs:
            leg.run(True)
        torch.cuda.synchronize()
        for leg in legs:
            leg.collect()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    summaries = {leg.name: leg.summary() for leg in legs}
    for s in summaries.values():
        frac = f"{100 * s['frac_of_peak']:.1f}% of peak, " if "frac_of_peak" in s else ""
        log(f"{s['name']:34s} {s['ms']:9.4f} ms x{s['reps']:<3d} {s['value']:10.2f} {s['unit']:10s} "
            f"({frac}{s['us_per_launch']:.2f} us/launch)")

    # ---- measured ceilings ------------------------------------------------------
    ceil = {}
    if "ceilings" in legs_wanted:
        ceil = {
            "launch_floor_us": {k.split("_")[-1]: summaries[k]["us_per_launch"]
                                for k in summaries if k.startswith("ceiling_empty_kernel_")},
            "stream_read_gbs": summaries["ceiling_stream_read_6713344B"]["value"],
            "stream_read_us_per_launch": summaries["ceiling_stream_read_6713344B"]["us_per_launch"],
            "stream_read_write_gbs": summaries["ceiling_stream_read_write_6713344B"]["value"],
            "stream_read_write_us_per_launch": summaries["ceiling_stream_read_write_6713344B"]["us_per_launch"],
            "mfma_i8_tops": max(s["value"] for k, s in summaries.items() if k.startswith("ceiling_mfma_i8_")),
            "mfma_f16_tflops": max(s["value"] for k, s in summaries.items() if k.startswith("ceiling_mfma_f16_")),
            "valu_ginstr_per_s": max(s["value"] for k, s in summaries.items()
                                     if k.startswith("ceiling_valu_mad_i24_")),
            "mfma_i8_with_24_valu_tops": summaries["ceiling_mix_i8_24valu_512x256"]["value"],
            "mfma_i8_with_33_valu_tops": summaries["ceiling_mix_i8_33valu_512x256"]["value"],
            "mfma_f16_with_14_valu_tflops": summaries["ceiling_mix_f16_14valu_512x256"]["value"],
            "lds_read_gbs": summaries["ceiling_lds_read_b128"]["value"],
            "lds_write_gbs": summaries["ceiling_lds_write_b128"]["value"],
            "how": "ceilings/ceilings.hip, timed in this run: empty kernels (1000 per graph) with 1x64 lanes and "
                   "with the decode GEMV's 512x256 grid; a cold read of 6,713,344 B per launch (80 buffers "
                   "rotated, the GEMV's grid), and the same with the GEMV's traffic split as it is (6,688,768 B "
                   "read, 12,288 bf16 written); back-to-back v_mfma_i32_32x32x32_i8 and, apart, "
                   "v_mfma_f32_32x32x16_f16 with 4 independent accumulators; back-to-back v_mad_i32_i24 in 8 "
                   "independent chains (best of two grid sizes); the MFMA loops with 24 or 33 (int8) and 14 (fp16) independent v_mad_i32_i24 per MFMA in "
                   "the same waves (the MMQs' instruction mixes); ds_read_b128 and ds_write_b128 by every "
                   "lane, bank-conflict free"}

        # each MMQ leg against the measured rate of the MFMA it runs on
        for s in summaries.values():
            k = s.get("kernel", "")
            c = (ceil["mfma_f16_tflops"] if k.startswith("q4k_mmq") else
                 ceil["mfma_i8_tops"] if k.startswith(("q2_0_mmq", "quantize_q8_1_kernel + q2_0_mmq")) else None)
            if c:
                s["frac_of_ceiling"] = round(s["value"] / c, 4)
            cm = (ceil["mfma_f16_with_14_valu_tflops"] if k.startswith("q4k_mmq") else
                  ceil["mfma_i8_with_33_valu_tops"] if k.startswith("q2_0_mmq") else None)
            if cm:
                s["frac_of_mix_ceiling"] = round(s["value"] / cm, 4)

    result = {"metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3), "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
              "config": {"workload": "decode GEMV m=1: Q2_0 qkvz n=12288 k=2048 group 128, 1000 calls per "
                                     "step, weight rotated through 80 copies (537 MB) so each call reads HBM",
                         "step": sorted(summaries)}}
    if "decode_gemv_m1" in summaries:
        s = summaries["decode_gemv_m1"]
        result["value"] = s["value"]
        result["roofline"] = {"bound": "hbm", "achieved": s["value"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": s["frac_of_peak"], "traffic": measured_traffic(TRAFFIC_DECODE),
                              "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                              "copy-calibrated)",
                              "kernel": s["kernel"], "us_per_launch": s["us_per_launch"],
                              "bytes_per_launch": DECODE_BYTES,
                              "warm_gbs": summaries.get("decode_gemv_m1_warm", {}).get("value")}
        if ceil:
            result["roofline"]["ceilings"] = ceil
            result["roofline"]["frac_of_ceiling"] = round(s["value"] / ceil["stream_read_write_gbs"], 4)
            result["roofline"]["ceiling_kernel"] = "stream_read_write_kernel"
    if "prefill_mmq_m2048" in summaries:
        s = summaries["prefill_mmq_m2048"]
        result["prefill"] = {"metric": "Q2_0 MMQ prefill int8 TOPS (2mnk / kernel time), m=2048 n=12288 k=2048",
                             "value": s["value"], "unit": "TOPS", "dtype": "i8",
                             "quantize_plus_mmq_tops": summaries["prefill_quantize_mmq_m2048"]["value"],
                             "roofline": {"bound": "mfma", "achieved": s["value"], "peak": INT8_PEAK_TOPS,
                                          "unit": "TOP/s", "frac": s["frac_of_peak"],
                                          "traffic": measured_traffic(TRAFFIC_MMQ),
                                          "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + "
                                                          "WRITE_SIZE, copy-calibrated)",
                                          "ops_per_launch": 2 * 2048 * 12288 * 2048,
                                          "algorithmic_bytes_per_launch": 61734912}}
        if ceil:
            result["prefill"]["roofline"]["frac_of_ceiling"] = round(s["value"] / ceil["mfma_i8_tops"], 4)
            result["prefill"]["roofline"]["frac_of_mix_ceiling"] = round(
                s["value"] / ceil["mfma_i8_with_33_valu_tops"], 4)
    result["legs"] = summaries

    # ---- CPU oracle baselines (rank 0, N = 1), on one pinned host core ----------
    if not args.no_cpu_baseline:
        log("oracle baselines on one host core")
        cb = cpu_baselines(ctx, args.cpu_seconds)
        if "decode_gemv_n12288_k2048" in cb:
            result["cpu_baseline"] = cb["decode_gemv_n12288_k2048"]
        if "prefill_qkvz_mmq_m2048" in cb and "prefill" in result:
            result["prefill"]["cpu_baseline"] = cb["prefill_qkvz_mmq_m2048"]
        result["cpu_baselines"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

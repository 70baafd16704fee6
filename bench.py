"""Benchmark of the packed low-bit weight-quantized matmul hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one pass of the whole hot path over one batch of synthetic
input, every leg on the current stream, each leg captured once into a HIP
graph and replayed between HIP events:
  decode   : 1000 x q2_0_gemv_vec, qkvz n=12288 k=2048 (m=1), the weight
             rotated through 80 copies (537 MB > the 256 MB Infinity Cache) so
             that every call streams its weight from HBM;
  verify   : q2_0_gemv_vec_batchm chain gate -> up -> silu_mul -> down,
             FFN [17408, 5120] / [5120, 17408], m in {2, 3, 4, 8}; and the same
             step with q2_0_gemv_gate_up_silu in place of the first three calls;
  prefill  : quantize_act_q8_1 + q2_0_mmq_gemm, qkvz n=12288 k=2048, m in
             {512, 2048}; and the bf16 fallback (dequant + dense GEMM) at m=512;
  ffn      : m=4096 FFN prefill, Q2_0 and Q4_K: quantize, gate and up MMQ
             (sharing the quantized input), silu_mul fused into the down
             projection's quantization, down MMQ;
  q4k      : Q4_K decode GEMV (m=1) on the FFN gate [17408, 5120] and down
             [5120, 17408] shapes, each weight rotated through 8 copies
             (401 MB); and the Q4_K weight quantizer on a bf16 [17408, 5120]
             weight (two input/output pairs alternate);
  copy     : (not in the default set) a plain 256 MiB device-to-device copy,
             the known-size reference for the HBM byte counters.
The JSON line reports the decode GEMV (the workload the headline metric is
quoted on) as `value`, with its roofline and the CPU oracle beside it; the
other legs are reported under "legs".  Inputs are resident in HBM before the
timed region starts.
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

DECODE_CALLS = 1000
DECODE_COPIES = 80
COPY_BYTES = 256 << 20
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
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--legs", default="decode,verify,prefill,ffn,q4k")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Leg:
    """A captured HIP graph plus its event timings.

    `keep` holds every tensor the captured kernels touch: the graph stores raw
    device pointers, and torch.cuda.graph() empties the allocator cache when a
    later capture begins, so a tensor without a live reference would be
    unmapped under an earlier graph."""

    def __init__(self, name, fn, keep, launches, work, unit, kernel, peak, bound, min_ms=2.0):
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
        scale = 1e9 if self.unit == "GB/s" else 1e12
        achieved = rate / scale
        return dict(name=self.name, ms=round(ms, 4), reps=self.reps, us_per_launch=round(per_launch_us, 3),
                    value=round(achieved, 2), unit=self.unit, kernel=self.kernel,
                    frac_of_peak=round(achieved / self.peak, 4), bound=self.bound)


def decode_leg(bq, dev, d):
    """1000 m=1 GEMV calls, weight rotated through DECODE_COPIES copies."""
    import torch
    n, k = d["n"], d["k"]
    w0 = torch.from_numpy(d["w"]).to(dev)
    wcopies = [w0] + [w0.clone() for _ in range(DECODE_COPIES - 1)]
    x = torch.from_numpy(d["act"][0].copy().view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.empty((n,), dtype=torch.bfloat16, device=dev)

    def fn():
        for i in range(DECODE_CALLS):
            bq.q2_0_gemv_vec(x, wcopies[i % DECODE_COPIES], y, n, k)

    bytes_per_call = w0.numel() + 2 * k + 2 * n
    leg = Leg("decode_gemv_m1", fn, wcopies + [x, y], DECODE_CALLS, DECODE_CALLS * bytes_per_call, "GB/s",
              "q2_0_gemv1_kernel", HBM_PEAK_GBS, "hbm")
    return leg, bytes_per_call


def verify_leg(bq, dev, W, act, m, H, I):
    import torch
    wg, wu, wd = W
    x = torch.from_numpy(np.ascontiguousarray(act[:m]).view(np.int16)).to(dev).view(torch.bfloat16)
    g_ = torch.empty((m, I), dtype=torch.bfloat16, device=dev)
    u_ = torch.empty((m, I), dtype=torch.bfloat16, device=dev)
    o_ = torch.empty((m, H), dtype=torch.bfloat16, device=dev)

    def fn():
        bq.q2_0_gemv_vec_batchm(x, wg, g_, m, I, H)
        bq.q2_0_gemv_vec_batchm(x, wu, u_, m, I, H)
        bq.silu_mul_bf16(g_, u_, g_, m * I)
        bq.q2_0_gemv_vec_batchm(g_, wd, o_, m, H, I)

    work = wg.numel() + wu.numel() + wd.numel() + m * (6 * H + 12 * I)
    kname = (f"q2_0_gemv_mfma_kernel<{m}> x3 + silu_mul" if m >= 4 else
             f"q2_0_gemvp_kernel<{m}> gate, up + silu_mul + q2_0_gemvm_kernel<{m}> down")
    return Leg(f"verify_ffn_m{m}", fn, [wg, wu, wd, x, g_, u_, o_], 4, work, "GB/s",
               kname, HBM_PEAK_GBS, "hbm")


def verify_fused_leg(bq, dev, W, act, m, H, I):
    """The same FFN step with gate, up and silu_mul fused into one launch."""
    import torch
    wg, wu, wd = W
    x = torch.from_numpy(np.ascontiguousarray(act[:m]).view(np.int16)).to(dev).view(torch.bfloat16)
    h_ = torch.empty((m, I), dtype=torch.bfloat16, device=dev)
    o_ = torch.empty((m, H), dtype=torch.bfloat16, device=dev)

    def fn():
        bq.q2_0_gemv_gate_up_silu(x, wg, wu, h_, m, I, H)
        bq.q2_0_gemv_vec_batchm(h_, wd, o_, m, H, I)

    work = wg.numel() + wu.numel() + wd.numel() + m * (2 * H + 4 * I)
    kname = (f"q2_0_gemv_mfma_kernel<{m}> gate+up+silu, q2_0_gemv_mfma_kernel<{m}> down" if m >= 4 else
             f"q2_0_gemvp_kernel<{m}> gate+up+silu, q2_0_gemvm_kernel<{m}> down")
    return Leg(f"verify_ffn_fused_m{m}", fn, [wg, wu, wd, x, h_, o_], 2, work, "GB/s",
               kname, HBM_PEAK_GBS, "hbm")


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
    legs = []
    for m in (512, 2048):
        x = torch.from_numpy(np.ascontiguousarray(p["act"][:m]).view(np.int16)).to(dev).view(torch.bfloat16)
        q8 = torch.empty((bq.q8_1_act_bytes(m, k),), dtype=torch.uint8, device=dev)
        y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        bq.quantize_act_q8_1(x, q8, m, k)
        legs.append(Leg(f"prefill_mmq_m{m}", lambda m=m, q8=q8, y=y: bq.q2_0_mmq_gemm(q8, w, y, m, n, k),
                        [w, q8, y], 1, 2.0 * m * n * k, "TOPS", "q2_0_mmq_kernel", INT8_PEAK_TOPS, "mfma"))
        legs.append(Leg(f"prefill_quantize_m{m}", lambda m=m, x=x, q8=q8: bq.quantize_act_q8_1(x, q8, m, k),
                        [x, q8], 1, 2 * m * k + bq.q8_1_act_bytes(m, k), "GB/s", "quantize_q8_1_kernel",
                        HBM_PEAK_GBS, "hbm"))
    m = 512
    x = torch.from_numpy(np.ascontiguousarray(p["act"][:m]).view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    scratch = torch.empty((n * k,), dtype=torch.bfloat16, device=dev)
    legs.append(Leg("fallback_dequant", lambda: bq.dequant_q2_0_to_bf16(w, scratch, n, k, 128), [w, scratch],
                    1, w.numel() + 2 * n * k, "GB/s", "dequant_q2_0_kernel", HBM_PEAK_GBS, "hbm"))
    legs.append(Leg("fallback_dense_gemm_m512", lambda: bq.dense_gemm_bf16(x, scratch, y, m, n, k),
                    [x, scratch, y], 1, 2.0 * m * n * k, "TOPS", "dense_gemm_bf16_kernel", BF16_PEAK_TFLOPS,
                    "mfma"))
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
    for fmt, key, gemm, kname in (("q2_0", "q2", bq.q2_0_mmq_gemm, "q2_0_mmq_kernel"),
                                  ("q4k", "q4k", bq.q4k_mmq_gemm, "q4k_mmq_kernel")):
        wg, wu, wd = (torch.from_numpy(F[key][name]).to(dev) for name in ("wg", "wu", "wd"))

        def ffn(wg=wg, wu=wu, wd=wd, gemm=gemm):
            bq.quantize_act_q8_1(x, q8a, m, H)
            gemm(q8a, wg, gate, m, I, H)
            gemm(q8a, wu, up, m, I, H)
            bq.silu_mul_quantize_q8_1(gate, up, q8h, m, I)
            gemm(q8h, wd, out, m, H, I)

        keep = [wg, wu, wd, x, q8a, q8h, gate, up, out]
        legs.append(Leg(f"ffn_prefill_{fmt}_m4096", ffn, keep, 5, 3 * 2.0 * m * H * I, "TOPS",
                        f"{kname} x3 + quantize + silu_mul_quantize", INT8_PEAK_TOPS, "mfma"))
        legs.append(Leg(f"ffn_gate_proj_{fmt}_m4096", lambda wg=wg, gemm=gemm: gemm(q8a, wg, gate, m, I, H),
                        keep, 1, 2.0 * m * H * I, "TOPS", kname, INT8_PEAK_TOPS, "mfma"))
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
    decode_ctx = None
    if "decode" in legs_wanted:
        d = inputs.decode_gemv()
        leg, bpc = decode_leg(bq, dev, d)
        legs.append(leg)
        decode_ctx = dict(d=d, bytes_per_call=bpc)
    if "verify" in legs_wanted:
        f = inputs.verify_ffn()
        W = tuple(torch.from_numpy(f[key]).to(dev) for key in ("wg", "wu", "wd"))
        for m in (2, 3, 4, 8):
            legs.append(verify_leg(bq, dev, W, f["act"], m, f["hidden"], f["inter"]))
        for m in (2, 3, 4, 8):
            legs.append(verify_fused_leg(bq, dev, W, f["act"], m, f["hidden"], f["inter"]))
    prefill_ctx = None
    if "prefill" in legs_wanted:
        prefill_ctx = inputs.prefill_qkvz()
        legs += prefill_legs(bq, dev, prefill_ctx)
    if "ffn" in legs_wanted:
        legs += ffn_legs(bq, dev, inputs.prefill_ffn())
    if "q4k" in legs_wanted:
        legs += q4k_legs(bq, dev, inputs.q4k_decode())
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
        log(f"{s['name']:28s} {s['ms']:9.4f} ms x{s['reps']:<3d} {s['value']:9.2f} {s['unit']:5s} "
            f"({100 * s['frac_of_peak']:.1f}% of peak, {s['us_per_launch']:.2f} us/launch)")

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
                              "bytes_per_launch": decode_ctx["bytes_per_call"]}
    if "prefill_mmq_m2048" in summaries:
        s = summaries["prefill_mmq_m2048"]
        result["prefill"] = {"metric": "Q2_0 MMQ prefill int8 TOPS (2mnk / kernel time), m=2048 n=12288 k=2048",
                             "value": s["value"], "unit": "TOPS", "dtype": "i8",
                             "roofline": {"bound": "mfma", "achieved": s["value"], "peak": INT8_PEAK_TOPS,
                                          "unit": "TOP/s", "frac": s["frac_of_peak"],
                                          "traffic": measured_traffic(TRAFFIC_MMQ),
                                          "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + "
                                                          "WRITE_SIZE, copy-calibrated)",
                                          "ops_per_launch": 2 * 2048 * 12288 * 2048,
                                          "algorithmic_bytes_per_launch": 61734912}}
    result["legs"] = summaries

    # ---- CPU oracle baselines (rank 0, N = 1), on one pinned host core ----------
    if not args.no_cpu_baseline:
        try:
            os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
        except Exception:
            pass
    if not args.no_cpu_baseline and "decode_gemv_m1" in summaries:
        import oracle
        d = decode_ctx["d"]
        calls, t_cpu = 0, 0.0
        while t_cpu < args.cpu_seconds and calls < 200:
            t1 = time.perf_counter()
            oracle.q2_0_gemv(d["act"], d["w"], 1, d["n"], d["k"])
            t_cpu += time.perf_counter() - t1
            calls += 1
        cpu_gbs = calls * decode_ctx["bytes_per_call"] / t_cpu / 1e9
        result["cpu_baseline"] = {"value": round(cpu_gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                                  "sample": f"{calls} decode GEMV calls (n=12288, k=2048) of the oracle, "
                                            f"{t_cpu:.1f} s on one pinned host core of {os.cpu_count()}"}
    # ---- CPU oracle baseline of the MMQ: 16 of the 2048 rows, all n -----------
    if not args.no_cpu_baseline and prefill_ctx is not None and "prefill" in result:
        import oracle
        p, rows = prefill_ctx, 16
        n, k = p["n"], p["k"]
        q8_rows, _ = oracle.quantize_act_q8_1(np.ascontiguousarray(p["act"][:rows]), rows, k)
        calls, t_cpu = 0, 0.0
        while t_cpu < args.cpu_seconds / 4 and calls < 50:
            t1 = time.perf_counter()
            oracle.q2_0_mmq(q8_rows, p["w"], rows, n, k)
            t_cpu += time.perf_counter() - t1
            calls += 1
        result["prefill"]["cpu_baseline"] = {
            "value": round(2.0 * rows * n * k * calls / t_cpu / 1e12, 6), "unit": "TOPS", "cores": 1,
            "kind": "oracle",
            "sample": f"{calls} oracle MMQ calls on {rows} of the 2048 activation rows (n=12288, k=2048; the "
                      f"oracle's cost is linear in rows), {t_cpu:.1f} s on one pinned host core of {os.cpu_count()}"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

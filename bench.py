"""Benchmark: bf16 -> MXFP8 quantize throughput on one MI355X.

A step is one pass of the quantize path over one batch: the rowwise and
columnwise planes of 64 MoE expert weights, each bf16 [2048, 7168] ~ N(0, 0.01),
in one grouped launch (1.88 GB in, 3.82 GB of algorithmic bytes per step).
That is the largest of the five workloads; the other four (a rowwise
[256, 1024] activation, the row + column [4096, 4096] weight with outliers and
zero / subnormal tiles, the fused RMSNorm + quantize at [8192, 8192], and the
fused op at decode [16, 7168] and prefill [65536, 7168]) are measured the same
way and reported under "configs".  Inputs are resident in HBM before timing
starts.  Workloads smaller than three times the 256 MB Infinity Cache rotate
over copies of their inputs and outputs, so every launch streams from HBM.

The timed steps are captured into one HIP graph and replayed once between
HIP events on the launch stream, so the figure is GPU time, not Python's
per-call overhead.  Each workload times at least 50 launches (20 for the
prefill), after at least 5 warm-up launches; every line but the headline
first replays its graph untimed for 25 ms, since the clocks ramp up over the
first milliseconds of work after an idle gap such as the capture.  After the
timed steps the headline launch is replayed for about 8 s ("sustained"; not
part of the value).  Every line but the headline reports the median of 5
timed replays.

Printed: one JSON line with GB/s of algorithmic bytes (input read once plus
every output written once), its fraction of the 8 TB/s HBM peak, the five
workloads, the other entry points, a plain device copy for context, and the
CPU oracle timed on bounded samples of every workload on this host.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--sustain S] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 matrix-core peak
MALL_BYTES = 256 << 20
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "mxfp8_block_scaled_02_amd", "csrc")
HEADLINE = "grouped_64x2048x7168"
# the headline step's one launch: 64 x (2048 / 32) x (7168 / 512) tiles
HEADLINE_KERNEL = "mx::mxfp8_quantize_kernel<mx::QuantArgs, false, true, false>/57344"

# the sources each kernel family is built from: a stored traffic figure is
# valid only while they are unchanged
KERNEL_SOURCES = {
    "mx::mxfp8_quantize_kernel": ("mx_device.h", "mx_kernels.h", "quantize.hip"),
    "mx::mxfp8_quantize_colt_kernel": ("mx_device.h", "mx_kernels.h", "quantize_colt.hip"),
    "mx::mxfp8_quantize_f32_kernel": ("mx_device.h", "mx_kernels.h", "quantize_f32.hip"),
    "mx::mxfp8_quantize_f32_colt_kernel": ("mx_device.h", "mx_kernels.h", "quantize_f32.hip"),
    "mx::mxfp8_rmsnorm_quantize_kernel": ("mx_device.h", "mx_kernels.h", "rmsnorm_quantize.hip"),
    "mx::mxfp8_dequantize_kernel": ("mx_device.h", "mx_kernels.h", "dequantize.hip"),
    "mx::mxfp8_gemm": ("mx_device.h", "mx_kernels.h", "gemm.hip"),
}


def sources_hash(kernel: str):
    """Hash of the sources of the kernel family a trace key belongs to."""
    for prefix, names in KERNEL_SOURCES.items():
        if kernel.startswith(prefix):
            h = hashlib.sha256()
            for name in names:
                with open(os.path.join(CSRC, name), "rb") as f:
                    h.update(name.encode() + f.read())
            return h.hexdigest()[:16]
    return None


def measured_traffic(kernel: str):
    """HBM bytes per launch of kernel from the committed counter runs, if they
    were taken on its current sources (else None)."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get("kernels", {}).get(kernel)
    if rec is None or rec.get("sources_hash") != sources_hash(kernel):
        return None
    return round(rec["bytes_per_launch"])


class Timed:
    """Times exactly `steps` calls of fn(i).

    The calls are captured once into a HIP graph (after `warmup` eager calls)
    and the graph is replayed once inside the timed region, so the time is
    the GPU's and not Python's per-call overhead.  HIP events on the replay
    stream bracket the replay; the host synchronizes on both sides."""

    def __init__(self, torch, eager=False, warm_ms=0.0, replays=1):
        self.torch = torch
        self.eager = eager
        self.warm_ms = warm_ms
        self.replays = replays

    def run(self, fn, steps, warmup, replays=None):
        """replays > 1 (default: the constructor's): the graph is replayed that
        many times, each timed on its own, and the median replay is reported
        (the events also count any host delay before a replay reaches the
        GPU, so one replay alone can read several times too long).  warm_ms: the graph is
        first replayed untimed until that much time has passed (the clocks
        ramp up over the first ten or so milliseconds of work after an idle
        gap, such as the capture itself).  Eager: both ignored."""
        torch = self.torch
        replays = self.replays if replays is None else replays
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        if self.eager:
            # plain launches (for counter collection, one dispatch per call)
            start = torch.cuda.Event(enable_timing=True)
            stop = torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            start.record()
            for i in range(steps):
                fn(i)
            stop.record()
            torch.cuda.synchronize()
            return start.elapsed_time(stop) / steps, time.perf_counter() - t0
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                fn(i)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        t_warm = time.perf_counter()
        while self.warm_ms > 0 and (time.perf_counter() - t_warm) * 1e3 < self.warm_ms:
            g.replay()
            torch.cuda.synchronize()
        times, wall = [], 0.0
        for _ in range(replays):
            start = torch.cuda.Event(enable_timing=True)
            stop = torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            start.record(stream)
            g.replay()
            stop.record(stream)
            torch.cuda.synchronize()
            wall += time.perf_counter() - t0
            times.append(start.elapsed_time(stop) / steps)
        del g
        return sorted(times)[len(times) // 2], wall


def rotation(per_set_bytes: int) -> int:
    return max(2, -(-3 * MALL_BYTES // max(per_set_bytes, 1)))


EAGER = False


def quant_bytes(r, c, rowwise, columnwise, in_bytes=2):
    return r * c * in_bytes + (r * c + r * c // 32 if rowwise else 0) + (r * c + (r // 32) * c if columnwise else 0)


def fused_bytes(r, c):
    return r * c * 2 + r * c * 2 + r * c + r * c // 32 + c * 2


def rec(ms, alg, elems, launches, **extra):
    gbs = alg / (ms * 1e-3) / 1e9
    out = {"ms_per_launch": round(ms, 5), "GB_s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
           "Gelem_s": round(elems / (ms * 1e-3) / 1e9, 2), "alg_bytes": alg, "launches_timed": launches}
    out.update(extra)
    return out


def sustained(torch, fn, seconds, per_graph=200):
    """fn replayed for about `seconds` in graphs of per_graph launches, the
    host waiting for each replay: the rate once clocks and caches have
    settled.  Outside the K timed steps; HIP events bracket all replays."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per_graph):
            fn(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    replays = 0
    t0 = time.perf_counter()
    start.record(stream)
    while replays == 0 or time.perf_counter() - t0 < seconds:
        g.replay()
        torch.cuda.synchronize()
        replays += 1
    stop.record(stream)
    torch.cuda.synchronize()
    launches = replays * per_graph
    del g
    return start.elapsed_time(stop) / launches, launches, time.perf_counter() - t0


def bench_headline(torch, mx, synth, steps, warmup, sustain_s=0.0):
    """The grouped row + column quantize of 64 expert weights: one launch a step."""
    dev = torch.device("cuda:0")
    xs = synth.workload(HEADLINE, device=dev)["xs"]
    r, c = xs[0].shape
    alg = len(xs) * quant_bytes(r, c, True, True)
    outs = mx.quantize_grouped(xs, True, True)
    fn = lambda i: mx.quantize_grouped(xs, True, True, outs=outs)
    ms, wall = Timed(torch, EAGER).run(fn, steps, warmup)
    res = {"ms": ms, "bytes": alg, "elems": 64 * r * c, "wall_s": wall, "shape": [r, c], "tensors": 64}
    if sustain_s > 0 and not EAGER:
        sms, n, swall = sustained(torch, fn, sustain_s)
        gbs = alg / (sms * 1e-3) / 1e9
        res["sustained"] = {"launches": n, "seconds": round(swall, 2), "ms_per_launch": round(sms, 5),
                            "GB_s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    del xs, outs
    return res


def bench_configs(torch, mx, synth, steps):
    """The other four workloads, each at least 50 launches (20 for the 65536-row
    prefill) after 5 warm-up launches and 25 ms of untimed graph replays; the
    median of 5 timed replays."""
    dev = torch.device("cuda:0")
    T = Timed(torch, EAGER, warm_ms=25.0, replays=5)   # untimed replays first: the clocks settle
    res = {}
    k_small = max(50, steps // 2)
    k_large = max(20, steps // 10)

    x = synth.workload("rowwise_256x1024", device=dev)["x"]
    r, c = x.shape
    alg = quant_bytes(r, c, True, False)
    n = min(rotation(alg), 512)
    xs = [x.clone() for _ in range(n)]
    outs = [mx.quantize(xi, True, False) for xi in xs]
    ms, _ = T.run(lambda i: mx.quantize(xs[i % n], True, False, out=outs[i % n]), k_small, 10)
    res["rowwise_256x1024"] = rec(ms, alg, r * c, k_small, rotating_sets=n, target_frac=0.70)
    del xs, outs

    x = synth.workload("rowcol_4096x4096", device=dev)["x"]
    r, c = x.shape
    alg = quant_bytes(r, c, True, True)
    n = rotation(alg)
    xs = [x.clone() for _ in range(n)]
    outs = [mx.quantize(xi, True, True) for xi in xs]
    ms, _ = T.run(lambda i: mx.quantize(xs[i % n], True, True, out=outs[i % n]), k_small, 10)
    res["rowcol_4096x4096"] = rec(ms, alg, r * c, k_small, rotating_sets=n, target_frac=0.70)
    del xs, outs

    w = synth.workload("rmsnorm_8192x8192", device=dev)
    r, c = w["x"].shape
    alg = fused_bytes(r, c)
    n = rotation(alg)
    xs = [w["x"]] + [w["x"].clone() for _ in range(n - 1)]
    os_ = [mx.rmsnorm_quantize(xi, w["gamma"], w["weight_offset"], w["eps"]) for xi in xs]
    ms, _ = T.run(lambda i: mx.rmsnorm_quantize(xs[i % n], w["gamma"], w["weight_offset"], w["eps"],
                                                out=os_[i % n]), k_small, 5)
    res["rmsnorm_8192x8192"] = rec(ms, alg, r * c, k_small, rotating_sets=n, target_frac=0.70)
    del w, xs, os_

    for name in ("rmsnorm_decode_16x7168", "rmsnorm_prefill_65536x7168"):
        w = synth.workload(name, device=dev)
        r, c = w["x"].shape
        alg = fused_bytes(r, c)
        # a small input rotates over copies; the prefill input alone is larger
        # than the Infinity Cache
        n = min(rotation(alg), 512) if alg < MALL_BYTES else 1
        xs = [w["x"]] + [w["x"].clone() for _ in range(n - 1)]
        os_ = [mx.rmsnorm_quantize(xi, w["gamma"], w["weight_offset"], w["eps"]) for xi in xs]
        k = k_small if r < 1024 else k_large
        ms, _ = T.run(lambda i: mx.rmsnorm_quantize(xs[i % n], w["gamma"], w["weight_offset"], w["eps"],
                                                    out=os_[i % n]), k, 5)
        res[name] = rec(ms, alg, r * c, k, rotating_sets=n)
        del w, xs, os_
    return res


def bench_other_rows(torch, mx, synth, steps):
    """The entry points outside the five workloads, each on its own input; the
    median of 5 timed replays."""
    dev = torch.device("cuda:0")
    res = {}
    T = Timed(torch, EAGER, warm_ms=25.0, replays=5)   # untimed replays first: the clocks settle

    x = synth.workload("rowwise_8192x7168", device=dev)["x"]
    r, c = x.shape
    alg = r * c * 3 + r * c // 32
    sets = rotation(alg)
    xs = [x.clone() for _ in range(sets)]
    del x
    outs = [mx.quantize(xi, True, False) for xi in xs]
    ms, _ = T.run(lambda i: mx.quantize(xs[i % sets], True, False, out=outs[i % sets]), max(steps // 4, 10), 3)
    res["rowwise_8192x7168"] = (ms, alg, r * c)
    del xs, outs

    x = synth.workload("rowcol_f32_4096x4096", device=dev)["x"]
    r, c = x.shape
    alg = r * c * 4 + 2 * r * c + r * c // 32 + (r // 32) * c
    sets = rotation(alg)
    xs = [x.clone() for _ in range(sets)]
    outs = [mx.quantize(xi, True, True) for xi in xs]
    ms, _ = T.run(lambda i: mx.quantize(xs[i % sets], True, True, out=outs[i % sets]), steps, 5)
    res["rowcol_f32_4096x4096"] = (ms, alg, r * c)
    outs = [mx.quantize(xi, True, True, columnwise_transposed=True) for xi in xs]
    ms, _ = T.run(lambda i: mx.quantize(xs[i % sets], True, True, out=outs[i % sets], columnwise_transposed=True),
                  steps, 5)
    res["rowcol_f32_4096x4096_transposed_columnwise"] = (ms, alg, r * c)
    del xs, outs

    # context: a plain device copy moving the 4096 x 4096 weight's volume
    sets = rotation(2 * (32 << 20))
    srcs = [torch.empty(32 << 20, dtype=torch.uint8, device=dev).fill_(1) for _ in range(sets)]
    dsts = [torch.empty_like(t) for t in srcs]
    ms, _ = T.run(lambda i: dsts[i % sets].copy_(srcs[i % sets]), steps, 5)
    res["context_device_copy_32MiB"] = (ms, 2 * (32 << 20), 0)
    del srcs, dsts

    # the 4096 x 4096 weight with both scale planes in padded allocations whose
    # rows are a pitch apart (136 and 4216 bytes instead of 128 and 4096):
    # same algorithmic bytes, written in place
    x = synth.workload("rowcol_4096x4096", device=dev)["x"]
    r, c = x.shape
    alg = r * c * 2 + 2 * r * c + r * c // 32 + (r // 32) * c
    sets = rotation(alg)
    xs = [x.clone() for _ in range(sets)]
    outs = []
    for _ in range(sets):
        _, sr = mx.padded_scale_plane(r, c, mx.ROWWISE, 128, 136, device=dev)
        _, sc = mx.padded_scale_plane(r, c, mx.COLUMNWISE, 4, 136, device=dev)
        outs.append(mx.MXFP8Planes(None, None, sr, sc))
    outs = [mx.quantize(xs[i], True, True, out=outs[i]) for i in range(sets)]
    ms, _ = T.run(lambda i: mx.quantize(xs[i % sets], True, True, out=outs[i % sets]), steps, 5)
    res["rowcol_4096x4096_padded_scales"] = (ms, alg, r * c)
    del xs, outs

    # the columnwise plane stored transposed ([cols, rows], the operand order
    # of the backward products): the same algorithmic bytes as both planes
    xs = [x.clone() for _ in range(sets)]
    outs = [mx.quantize(xi, True, True, columnwise_transposed=True) for xi in xs]
    ms, _ = T.run(lambda i: mx.quantize(xs[i % sets], True, True, out=outs[i % sets], columnwise_transposed=True),
                  steps, 5)
    res["rowcol_4096x4096_transposed_columnwise"] = (ms, alg, r * c)
    del xs, outs
    ws = synth.workload(HEADLINE, device=dev)["xs"]
    wr, wc = ws[0].shape
    outs = mx.quantize_grouped(ws, True, True, columnwise_transposed=True)
    ms, _ = T.run(lambda i: mx.quantize_grouped(ws, True, True, outs=outs, columnwise_transposed=True),
                  max(20, steps // 10), 3)
    res[HEADLINE + "_transposed_columnwise"] = (ms, len(ws) * quant_bytes(wr, wc, True, True), len(ws) * wr * wc)
    del ws, outs

    p = mx.quantize(x, True, True)
    for axis, q, s in ((0, p.rowwise_data, p.rowwise_scale), (1, p.columnwise_data, p.columnwise_scale)):
        alg = r * c + s.numel() + r * c * 4
        sets = rotation(alg)
        qs = [(q.clone(), s.clone()) for _ in range(sets)]
        outs = [mx.dequantize(qi, si, axis) for qi, si in qs]
        ms, _ = T.run(lambda i: mx.dequantize(qs[i % sets][0], qs[i % sets][1], axis, out=outs[i % sets]),
                      steps, 5)
        res["dequantize_f32_%s_4096x4096" % ("row" if axis == 0 else "col")] = (ms, alg, r * c)
        del qs, outs
    out = {k: {"ms_per_launch": round(ms, 5), "GB_s": round(b / (ms * 1e-3) / 1e9, 1),
               "frac_hbm": round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "Gelem_s": round(e / (ms * 1e-3) / 1e9, 2), "alg_bytes": b}
           for k, (ms, b, e) in res.items()}
    out.update(bench_gemm(torch, mx, steps, synth))
    return out


def bench_gemm(torch, mx, steps, synth=None):
    """The MXFP8 product of a quantized activation and a quantized weight:
    TFLOP/s (2 M N K per launch) against the dense fp8 matrix-core peak."""
    dev = torch.device("cuda:0")
    T = Timed(torch, EAGER, warm_ms=25.0)   # untimed replays first: the clocks settle
    res = {}
    # 4096 x 4096 x 11008: an MLP down projection, K not a multiple of 512;
    # 256 x 2048 x 7168: 256 tokens through one 2048 x 7168 expert weight;
    # 64 x 28672 x 7168: 64 tokens through a fused gate and up projection
    # (two 14336 x 7168 weights), a wide weight under a few rows
    # "_mfma_scales": both operands' scales in the MFMA order (K % 512 == 0)
    for M, N, K, order in ((8192, 8192, 8192, "row"), (8192, 8192, 8192, "mfma"),
                           (1024, 7168, 7168, "row"), (1024, 7168, 7168, "mfma"),
                           (4096, 4096, 11008, "row"), (256, 2048, 7168, "row"),
                           (64, 28672, 7168, "row"),
                           (128, 7168, 7168, "row"), (128, 7168, 7168, "mfma"),
                           (16, 7168, 7168, "row"), (16, 7168, 7168, "mfma")):
        g = torch.Generator(device=dev).manual_seed(M + N + K)
        a = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
        b = (torch.randn((N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16)
        pa = mx.quantize(a, True, False, scale_order=order)
        pb = mx.quantize(b, True, False, scale_order=order)
        del a, b
        # the weight rotates over copies that together exceed the Infinity
        # Cache, so every launch reads B from HBM, as a layer's weight is
        sets = rotation(N * K + N * K // 32)
        bs = [(pb.rowwise_data.clone(), pb.rowwise_scale.clone()) for _ in range(sets)]
        del pb
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        fn = lambda i: mx.gemm(pa.rowwise_data, pa.rowwise_scale, bs[i % sets][0], bs[i % sets][1],
                               torch.bfloat16, out=out)
        # the median of 5 replays: one replay of a few launches of the large
        # products varies by several percent with the clock
        ms, _ = T.run(fn, max(steps // 4, 10), 3, replays=5)
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        rec = {"ms_per_launch": round(ms, 5), "TFLOP_s": round(tf, 1),
               "frac_mfma_fp8": round(tf / FP8_MFMA_PEAK_TFLOPS, 4)}
        if M <= 512:
            # a few rows against a large weight: bound by streaming the planes
            # of B (and A) once and writing the output
            alg = (M + N) * K * (1 + 1 / 32) + M * N * 2
            rec.update({"alg_bytes": int(alg), "GB_s": round(alg / (ms * 1e-3) / 1e9, 1),
                        "frac_hbm": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
        res["gemm_bf16out_%dx%dx%d%s" % (M, N, K, "_mfma_scales" if order == "mfma" else "")] = rec
        del bs, pa, out

    # the grouped product of an MoE layer in decode: the 64 expert weights
    # [2048, 7168] of the grouped quantize, 16 tokens each, one launch; the
    # weights (940 MB) exceed the Infinity Cache, so each launch reads them
    # from HBM
    ws = synth.workload(HEADLINE, device=dev)["xs"]
    E, (N, K), tok = len(ws), ws[0].shape, 16
    pw = mx.quantize_grouped(ws, True, False)
    del ws
    g = torch.Generator(device=dev).manual_seed(7)
    pa = [mx.quantize(torch.randn((tok, K), generator=g, device=dev).to(torch.bfloat16), True, False)
          for _ in range(E)]
    outs = [torch.empty((tok, N), dtype=torch.bfloat16, device=dev) for _ in range(E)]
    args = ([p.rowwise_data for p in pa], [p.rowwise_scale for p in pa], [p.rowwise_data for p in pw],
            [p.rowwise_scale for p in pw])
    ms, _ = T.run(lambda i: mx.gemm_grouped(*args, torch.bfloat16, outs=outs), max(steps // 4, 20), 3, replays=5)
    alg = E * ((tok + N) * K * (1 + 1 / 32) + 2 * tok * N)
    tf = 2.0 * E * tok * N * K / (ms * 1e-3) / 1e12
    res["gemm_grouped_moe_64_experts_16x2048x7168"] = {
        "ms_per_launch": round(ms, 5), "TFLOP_s": round(tf, 1), "frac_mfma_fp8": round(tf / FP8_MFMA_PEAK_TFLOPS, 4),
        "alg_bytes": int(alg), "GB_s": round(alg / (ms * 1e-3) / 1e9, 1),
        "frac_hbm": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del pw, pa, outs, args
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(torch, synth, min_s=0.75, dev="cuda:0"):
    """The oracle on bounded samples of every workload, with all host threads
    (OpenMP over rows, and over tensors for the experts) and with one thread.

    Each sample is cut from the same seeded input the GPU quantizes (drawn on
    the device, copied back).  Each leg repeats the sample until min_s seconds
    have passed; rates are GB/s and Gelem/s of the same algorithmic bytes as
    the GPU figures.  About 15 s of CPU work in all."""
    import oracle
    dev = torch.device(dev)
    cores = oracle.max_threads()

    def leg(fn, alg, elems, threads, what, limit=min_s):
        oracle.set_threads(threads)
        try:
            reps, t0 = 0, time.perf_counter()
            while True:
                fn()
                reps += 1
                el = time.perf_counter() - t0
                if el >= limit or reps >= 10000:
                    break
        finally:
            oracle.set_threads(cores)
        return {"GB_s": round(alg * reps / el / 1e9, 4), "Gelem_s": round(elems * reps / el / 1e9, 5),
                "threads": threads, "sample": "%s, %d passes in %.2f s" % (what, reps, el)}

    def quant(bits, row, col):
        def fn():
            if row:
                oracle.quantize_rowwise(bits)
            if col:
                oracle.quantize_colwise(bits)
        return fn

    def fused(w, bits):
        gb = synth.bf16_bits(w["gamma"])
        return lambda: oracle.rmsnorm_quantize(bits, gb, w["weight_offset"], w["eps"])

    out = {}
    x = synth.bf16_bits(synth.workload("rowwise_256x1024", device=dev)["x"])
    r, c = x.shape
    out["rowwise_256x1024"] = [leg(quant(x, True, False), quant_bytes(r, c, True, False), r * c, t,
                                   "the whole [256, 1024] tensor") for t in (cores, 1)]

    x = synth.bf16_bits(synth.workload("rowcol_4096x4096", device=dev)["x"])
    legs = []
    for t, rows in ((cores, 4096), (1, 1024)):
        xs = x[:rows]
        legs.append(leg(quant(xs, True, True), quant_bytes(rows, 4096, True, True), rows * 4096, t,
                        "rows 0..%d of the [4096, 4096] weight, both planes" % rows))
    out["rowcol_4096x4096"] = legs

    xs = synth.workload(HEADLINE, device=dev)["xs"]
    legs = []
    for t, n_exp, rows in ((cores, 8, 2048), (1, 1, 1024)):
        bits = [synth.bf16_bits(e[:rows]) for e in xs[:n_exp]]
        fn = (lambda b=bits: [quant(e, True, True)() for e in b])
        legs.append(leg(fn, n_exp * quant_bytes(rows, 7168, True, True), n_exp * rows * 7168, t,
                        "%d of the 64 expert weights (rows 0..%d each), both planes" % (n_exp, rows)))
    out[HEADLINE] = legs
    del xs

    for name, samples in (("rmsnorm_8192x8192", ((cores, 4096), (1, 512))),
                          ("rmsnorm_decode_16x7168", ((cores, 16), (1, 16))),
                          ("rmsnorm_prefill_65536x7168", ((cores, 8192), (1, 512)))):
        w = synth.workload(name, device=dev)
        R, C = w["x"].shape
        legs = []
        for t, rows in samples:
            bits = synth.bf16_bits(w["x"][:rows])
            legs.append(leg(fused(w, bits), fused_bytes(rows, C), rows * C, t,
                            "rows 0..%d of [%d, %d], normed + rowwise plane" % (rows, R, C)))
        out[name] = legs
        del w

    head = out[HEADLINE]
    return {"value": head[0]["GB_s"], "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": head[0]["sample"] + " (the headline workload)",
            "value_1_thread": head[1]["GB_s"], "sample_1_thread": head[1]["sample"],
            "cpu_model": cpu_model(),
            "per_config": {k: {"all_threads": v[0], "one_thread": v[1]} for k, v in out.items()}}


def short_kernel_name(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0]


def trace_summary(trace_csv: str) -> str:
    """Per-kernel launch durations from a rocprofv3 --kernel-trace CSV (text)."""
    import csv
    import collections
    agg = collections.defaultdict(list)
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if "mx::" not in name and "copy" not in name.lower():
                continue
            key = (short_kernel_name(name), int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]))
            agg[key].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines = ["%-80s %10s %6s %10s %10s %10s %10s %10s" % ("kernel", "workgroups", "calls", "mean_us",
                                                          "p10_us", "median_us", "p90_us", "min_us")]
    for (name, wgs), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        v.sort()
        lines.append("%-80s %10d %6d %10.3f %10.3f %10.3f %10.3f %10.3f" % (
            name[-80:], wgs, len(v), sum(v) / len(v) / 1e3, percentile(v, 10) / 1e3, v[len(v) // 2] / 1e3,
            percentile(v, 90) / 1e3, v[0] / 1e3))
    return "\n".join(lines)


def percentile(sorted_values, q):
    """The q-th percentile of a sorted list (nearest rank)."""
    k = max(0, min(len(sorted_values) - 1, -(-q * len(sorted_values) // 100) - 1))
    return sorted_values[k]


def counter_bytes(counter_csv: str, counter: str):
    """{(kernel, workgroups): [KiB per dispatch]} for one counter."""
    import csv
    import collections
    out = collections.defaultdict(list)
    with open(counter_csv) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            key = (short_kernel_name(r["Kernel_Name"]),
                   int(r["Grid_Size"]) // int(r["Workgroup_Size"]))
            out[key].append(float(r["Counter_Value"]))
    return out


def traffic_summary(fetch_csv: str, write_csv: str, copy_bytes: int = 256 << 20):
    """HBM bytes per launch of the quantize kernel, each counter scaled by what
    it reads for a plain device copy of copy_bytes (the largest copy kernel
    dispatch in the same run)."""
    fetch = counter_bytes(fetch_csv, "FETCH_SIZE")
    write = counter_bytes(write_csv, "WRITE_SIZE")
    # the runtime's device-to-device copy kernel; its largest dispatch is the
    # 256 MiB calibration copy
    copy_f = max(max(v) for k, v in fetch.items() if "copyBuffer" in k[0])
    copy_w = max(max(v) for k, v in write.items() if "copyBuffer" in k[0])
    f_scale = copy_bytes / (copy_f * 1024.0)
    w_scale = copy_bytes / (copy_w * 1024.0)
    res = {}
    for key, v in fetch.items():
        if "mx::" not in key[0] or key not in write:
            continue
        fb = sum(v) / len(v) * 1024.0 * f_scale
        wb = sum(write[key]) / len(write[key]) * 1024.0 * w_scale
        res["%s/%d" % key] = {"fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb,
                              "sources_hash": sources_hash(key[0])}
    return {"fetch_scale": f_scale, "write_scale": w_scale, "kernels": res}


def main():
    if len(sys.argv) > 2 and sys.argv[1] == "--trace-summary":
        print(trace_summary(sys.argv[2]))
        return
    if len(sys.argv) > 3 and sys.argv[1] == "--traffic-summary":
        res = traffic_summary(sys.argv[2], sys.argv[3])
        print(json.dumps(res, indent=1))
        if "--write" in sys.argv:
            path = os.path.join(PROFILES, "traffic.json")
            old = {}
            if os.path.exists(path):
                with open(path) as f:
                    old = json.load(f).get("kernels", {})
            # keep the records of kernels this run did not launch, unless their
            # sources changed since (then no record of them is current)
            old = {k: v for k, v in old.items() if v.get("sources_hash") == sources_hash(k.split("/")[0])}
            old.update(res["kernels"])
            res["kernels"] = old
            with open(path, "w") as f:
                json.dump(res, f, indent=1)
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-rows", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time plain launches instead of one graph replay (counter runs)")
    ap.add_argument("--sustain", type=float, default=8.0,
                    help="after the timed steps, replay the headline launch for this many "
                         "seconds and report the settled rate (0: skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB device copy, the reference that "
                         "scales HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path shards rows with no "
              "communication, so it runs and is reported per GPU (--gpus 1).", file=sys.stderr)
        sys.exit(2)

    global EAGER
    EAGER = args.eager
    import torch
    import mxfp8_block_scaled_02_amd as mx
    from mxfp8_block_scaled_02_amd import synth
    mx.lib()

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    main_run = bench_headline(torch, mx, synth, args.steps, args.warmup, args.sustain)
    ms = main_run["ms"]
    gbs = main_run["bytes"] / (ms * 1e-3) / 1e9
    line = {
        "metric": "bf16\u2192MXFP8 quantize GB/s (frac of MI355X HBM peak) + Gelem/s, 1 GPU",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": HEADLINE, "tensors": main_run["tensors"], "shape": main_run["shape"],
                   "planes": ["rowwise", "columnwise"], "alg_bytes_per_step": main_run["bytes"],
                   "launches_per_step": 1},
        "Gelem_s": round(main_run["elems"] / (ms * 1e-3) / 1e9, 2),
        # one launch per step, so the step time is the dominant kernel's
        # average launch duration
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(HEADLINE_KERNEL), "kernel": HEADLINE_KERNEL},
    }
    if "sustained" in main_run:
        line["sustained"] = main_run["sustained"]
    if not args.no_other_rows:
        line["configs"] = bench_configs(torch, mx, synth, args.steps)
        line["other_entry_points"] = bench_other_rows(torch, mx, synth, max(args.steps // 2, 20))
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(torch, synth)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

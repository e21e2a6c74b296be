"""Benchmark: bf16 -> MXFP8 quantize throughput on one MI355X.

A step is one pass of the quantize path over one batch: the rowwise and
columnwise planes of the bf16 weight [4096, 4096] (N(0, 0.02) with 0.1%
outliers x1000, 1% zero and 1% subnormal 32x32 tiles) from a single read.
Inputs are resident in HBM before timing starts.  The step rotates over
enough copies of input and outputs that the working set exceeds the 256 MB
Infinity Cache, so every step streams from HBM.

The timed steps are captured into one HIP graph and replayed once between
HIP events, so the figure is GPU time, not Python's per-call overhead.

Printed: one JSON line with GB/s of algorithmic bytes (input read once plus
every output written once), its fraction of the 8 TB/s HBM peak, the other
entry points measured the same way on their workloads, a plain device copy
of the same byte count for context, and the CPU oracle timed on a bounded
sample on this host.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
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


# the sources the headline quantize kernel is built from
QUANTIZE_SOURCES = ("mx_device.h", "mx_kernels.h", "quantize.hip")


def kernel_source_hash() -> str:
    """Hash of the quantize kernel's sources: stored traffic figures are valid
    only while it matches."""
    h = hashlib.sha256()
    for name in QUANTIZE_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed counter runs, if they were taken
    on the current kernel sources (else None)."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    if data.get("source_hash") != kernel_source_hash():
        return None
    rec = data.get("kernels", {}).get(workload)
    return None if rec is None else round(rec["bytes_per_launch"])


class Timed:
    """Times exactly `steps` calls of fn(i).

    The calls are captured once into a HIP graph (after `warmup` eager calls)
    and the graph is replayed once inside the timed region, so the time is
    the GPU's and not Python's per-call overhead.  HIP events on the replay
    stream bracket the replay; the host synchronizes on both sides."""

    def __init__(self, torch, eager=False):
        self.torch = torch
        self.eager = eager

    def run(self, fn, steps, warmup):
        torch = self.torch
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
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record(stream)
        g.replay()
        stop.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = start.elapsed_time(stop) / steps
        del g
        return ms, wall


def rotation(per_set_bytes: int) -> int:
    return max(2, -(-3 * MALL_BYTES // max(per_set_bytes, 1)))


EAGER = False


def bench_rowcol(torch, mx, synth, steps, warmup):
    dev = torch.device("cuda:0")
    x = synth.workload("rowcol_4096x4096", device=dev)["x"]
    rows, cols = x.shape
    alg = rows * cols * 2 + 2 * rows * cols + rows * cols // 32 + (rows // 32) * cols
    sets = rotation(alg)
    xs = [x.clone() for _ in range(sets)]
    outs = [mx.quantize(xi, True, True) for xi in xs]
    fn = lambda i: mx.quantize(xs[i % sets], True, True, out=outs[i % sets])
    ms, wall = Timed(torch, EAGER).run(fn, steps, warmup)
    return {"ms": ms, "bytes": alg, "elems": rows * cols, "sets": sets, "wall_s": wall}


def bench_other_rows(torch, mx, synth, steps):
    """Each remaining entry point on its own workload (fewer steps)."""
    dev = torch.device("cuda:0")
    res = {}
    T = Timed(torch, EAGER)

    x = synth.workload("rowwise_256x1024", device=dev)["x"]
    r, c = x.shape
    alg = r * c * 3 + r * c // 32
    sets = rotation(alg) if alg * rotation(alg) < (1 << 31) else 1
    xs = [x.clone() for _ in range(min(sets, 512))]
    outs = [mx.quantize(xi, True, False) for xi in xs]
    n = len(xs)
    ms, _ = T.run(lambda i: mx.quantize(xs[i % n], True, False, out=outs[i % n]), steps, 10)
    res["rowwise_256x1024"] = (ms, alg, r * c)

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

    w = synth.workload("rmsnorm_8192x8192", device=dev)
    r, c = w["x"].shape
    alg = r * c * 2 + r * c * 2 + r * c + r * c // 32 + c * 2
    sets = rotation(alg)
    xs = [w["x"].clone() for _ in range(sets)]
    os_ = [mx.rmsnorm_quantize(xi, w["gamma"], w["weight_offset"], w["eps"]) for xi in xs]
    ms, _ = T.run(lambda i: mx.rmsnorm_quantize(xs[i % sets], w["gamma"], w["weight_offset"], w["eps"],
                                                out=os_[i % sets]), max(steps // 4, 5), 3)
    res["rmsnorm_8192x8192"] = (ms, alg, r * c)
    del w, xs, os_

    xs = synth.workload("grouped_64x2048x7168", device=dev)["xs"]
    r, c = xs[0].shape
    alg = len(xs) * (r * c * 2 + 2 * r * c + r * c // 32 + (r // 32) * c)
    outs = mx.quantize_grouped(xs, True, True)
    ms, _ = T.run(lambda i: mx.quantize_grouped(xs, True, True, outs=outs), max(steps // 10, 5), 2)
    res["grouped_64x2048x7168"] = (ms, alg, len(xs) * r * c)
    del xs, outs

    for name in ("rmsnorm_decode_16x7168", "rmsnorm_prefill_65536x7168"):
        w = synth.workload(name, device=dev)
        r, c = w["x"].shape
        alg = r * c * 2 + r * c * 2 + r * c + r * c // 32 + c * 2
        # a small input rotates over copies like the small quantize line; the
        # prefill input alone is larger than the Infinity Cache
        n = min(rotation(alg), 512) if alg < MALL_BYTES else 1
        xs = [w["x"]] + [w["x"].clone() for _ in range(n - 1)]
        os_ = [mx.rmsnorm_quantize(xi, w["gamma"], w["weight_offset"], w["eps"]) for xi in xs]
        k = steps if r < 1024 else max(steps // 10, 5)
        ms, _ = T.run(lambda i: mx.rmsnorm_quantize(xs[i % n], w["gamma"], w["weight_offset"], w["eps"],
                                                    out=os_[i % n]), k, 3)
        res[name] = (ms, alg, r * c)
        del w, xs, os_

    x = synth.workload("rowcol_f32_4096x4096", device=dev)["x"]
    r, c = x.shape
    alg = r * c * 4 + 2 * r * c + r * c // 32 + (r // 32) * c
    sets = rotation(alg)
    xs = [x.clone() for _ in range(sets)]
    outs = [mx.quantize(xi, True, True) for xi in xs]
    ms, _ = T.run(lambda i: mx.quantize(xs[i % sets], True, True, out=outs[i % sets]), steps, 5)
    res["rowcol_f32_4096x4096"] = (ms, alg, r * c)
    del xs, outs

    # context: a plain device copy moving the row+column step's input volume
    sets = rotation(2 * (32 << 20))
    srcs = [torch.empty(32 << 20, dtype=torch.uint8, device=dev).fill_(1) for _ in range(sets)]
    dsts = [torch.empty_like(t) for t in srcs]
    ms, _ = T.run(lambda i: dsts[i % sets].copy_(srcs[i % sets]), steps, 5)
    res["context_device_copy_32MiB"] = (ms, 2 * (32 << 20), 0)
    del srcs, dsts

    # the headline workload with both scale planes in padded allocations whose
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
    out.update(bench_gemm(torch, mx, steps))
    return out


def bench_gemm(torch, mx, steps):
    """The MXFP8 product of a quantized activation and a quantized weight:
    TFLOP/s (2 M N K per launch) against the dense fp8 matrix-core peak."""
    dev = torch.device("cuda:0")
    T = Timed(torch, EAGER)
    res = {}
    # 4096 x 4096 x 11008: an MLP down projection, K not a multiple of 512
    for M, N, K in ((8192, 8192, 8192), (1024, 7168, 7168), (4096, 4096, 11008), (128, 7168, 7168),
                    (16, 7168, 7168)):
        g = torch.Generator(device=dev).manual_seed(M + N + K)
        a = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
        b = (torch.randn((N, K), generator=g, device=dev) * 0.02).to(torch.bfloat16)
        pa, pb = mx.quantize(a, True, False), mx.quantize(b, True, False)
        del a, b
        # the weight rotates over copies that together exceed the Infinity
        # Cache, so every launch reads B from HBM, as a layer's weight is
        sets = rotation(N * K + N * K // 32)
        bs = [(pb.rowwise_data.clone(), pb.rowwise_scale.clone()) for _ in range(sets)]
        del pb
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        fn = lambda i: mx.gemm(pa.rowwise_data, pa.rowwise_scale, bs[i % sets][0], bs[i % sets][1],
                               torch.bfloat16, out=out)
        ms, _ = T.run(fn, max(steps // 4, 10), 3)
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        rec = {"ms_per_launch": round(ms, 5), "TFLOP_s": round(tf, 1),
               "frac_mfma_fp8": round(tf / FP8_MFMA_PEAK_TFLOPS, 4)}
        if M <= 128:
            # a few rows against a large weight: bound by streaming the planes
            # of B (and A) once and writing the output
            alg = (M + N) * K * (1 + 1 / 32) + M * N * 2
            rec.update({"alg_bytes": int(alg), "GB_s": round(alg / (ms * 1e-3) / 1e9, 1),
                        "frac_hbm": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
        res["gemm_bf16out_%dx%dx%d" % (M, N, K)] = rec
        del bs, pa, out
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


def cpu_baseline(synth, target_s=12.0, single_s=6.0):
    """The oracle on full passes of the headline weight: all host threads for
    about target_s, then one thread for about single_s."""
    import oracle
    x = synth.workload("rowcol_4096x4096")["x"]
    bits = synth.bf16_bits(x)
    rows, cols = bits.shape
    alg = rows * cols * 2 + 2 * rows * cols + rows * cols // 32 + (rows // 32) * cols

    def passes(limit_s):
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.quantize_rowwise(bits)
            oracle.quantize_colwise(bits)
            reps += 1
            el = time.perf_counter() - t0
            if el >= limit_s or reps >= 1000:
                return reps, el

    cores = oracle.max_threads()
    reps, el = passes(target_s)
    oracle.set_threads(1)
    try:
        reps1, el1 = passes(single_s)
    finally:
        oracle.set_threads(cores)
    return {"value": round(alg * reps / el / 1e9, 3), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": "%d passes of the full 4096x4096 weight, rowwise + columnwise planes, %.1f s"
                      % (reps, el),
            "value_1_thread": round(alg * reps1 / el1 / 1e9, 4),
            "sample_1_thread": "%d passes, %.1f s" % (reps1, el1),
            "cpu_model": cpu_model()}


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
    lines = ["%-60s %10s %6s %10s %10s %10s %10s %10s" % ("kernel", "workgroups", "calls", "mean_us",
                                                          "p10_us", "median_us", "p90_us", "min_us")]
    for (name, wgs), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        v.sort()
        lines.append("%-60s %10d %6d %10.3f %10.3f %10.3f %10.3f %10.3f" % (
            name[-60:], wgs, len(v), sum(v) / len(v) / 1e3, percentile(v, 10) / 1e3, v[len(v) // 2] / 1e3,
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
        res["%s/%d" % key] = {"fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb}
    return {"fetch_scale": f_scale, "write_scale": w_scale, "kernels": res}


def main():
    if len(sys.argv) > 2 and sys.argv[1] == "--trace-summary":
        print(trace_summary(sys.argv[2]))
        return
    if len(sys.argv) > 3 and sys.argv[1] == "--traffic-summary":
        res = traffic_summary(sys.argv[2], sys.argv[3])
        res["source_hash"] = kernel_source_hash()
        res["hashed_sources"] = list(QUANTIZE_SOURCES)
        print(json.dumps(res, indent=1))
        if "--write" in sys.argv:
            with open(os.path.join(PROFILES, "traffic.json"), "w") as f:
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

    main_run = bench_rowcol(torch, mx, synth, args.steps, args.warmup)
    ms = main_run["ms"]
    gbs = main_run["bytes"] / (ms * 1e-3) / 1e9
    # the row+column launch on the 4096 x 4096 weight: (4096/32) x (4096/512) tiles
    traffic = measured_traffic("mx::mxfp8_quantize_kernel<mx::QuantArgs, true>/1024")
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
        "config": {"workload": "rowcol_4096x4096", "shape": [4096, 4096],
                   "planes": ["rowwise", "columnwise"], "alg_bytes_per_step": main_run["bytes"],
                   "rotating_sets": main_run["sets"]},
        "Gelem_s": round(main_run["elems"] / (ms * 1e-3) / 1e9, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic},
    }
    if not args.no_other_rows:
        line["other_entry_points"] = bench_other_rows(torch, mx, synth, max(args.steps // 2, 20))
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(synth)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

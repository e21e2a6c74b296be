"""The benchmark's host logic, without a GPU: algorithmic byte counts, the
percentile used in trace summaries, the trace and counter parsers, and the
refusal to run on more than one GPU."""
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_of_the_five_workloads():
    # input read once, every output written once: 1 B per element per data
    # plane, 1/32 B per scale plane, 2 B per normed element, 2 B per gamma
    assert bench.quant_bytes(256, 1024, True, False) == 794_624
    assert bench.quant_bytes(4096, 4096, True, True) == 68_157_440
    assert bench.fused_bytes(8192, 8192) == 337_657_856
    assert 64 * bench.quant_bytes(2048, 7168, True, True) == 3_816_816_640
    assert bench.fused_bytes(16, 7168) == 591_360
    assert bench.fused_bytes(65536, 7168) == 2_363_504_640
    # a float32 input reads 4 B per element
    assert bench.quant_bytes(4096, 4096, True, True, in_bytes=4) == 68_157_440 + 2 * 4096 * 4096


def test_percentile_is_nearest_rank():
    v = list(range(1, 101))
    assert bench.percentile(v, 10) == 10 and bench.percentile(v, 50) == 50
    assert bench.percentile(v, 90) == 90 and bench.percentile(v, 100) == 100
    assert bench.percentile([7], 10) == 7


def test_trace_summary(tmp_path):
    csv = tmp_path / "kernel_trace.csv"
    rows = ["Kernel_Name,Grid_Size_X,Workgroup_Size_X,Start_Timestamp,End_Timestamp"]
    for i, d in enumerate([1000, 3000, 2000, 4000, 5000]):
        rows.append('"void mx::(anonymous namespace)::mxfp8_quantize_kernel<mx::QuantArgs, true>(mx::QuantArgs)",'
                    "262144,256,%d,%d" % (10 * i * 1000, 10 * i * 1000 + d))
    rows.append('"other_kernel(int)",64,64,0,100')
    csv.write_text("\n".join(rows) + "\n")
    out = bench.trace_summary(str(csv)).splitlines()
    assert len(out) == 2
    f = out[1].split()
    assert f[0] == "mx::mxfp8_quantize_kernel<mx::QuantArgs," and f[1] == "true>"
    wgs, calls, mean, p10, med = int(f[2]), int(f[3]), float(f[4]), float(f[5]), float(f[6])
    assert (wgs, calls) == (1024, 5)
    assert mean == pytest.approx(3.0) and p10 == pytest.approx(1.0) and med == pytest.approx(3.0)


def test_traffic_summary_scales_by_the_copy(tmp_path):
    # the counters read half of a copy's fetched bytes and all of its written
    # bytes: the scale factors recover the copy's known size, and a kernel's
    # bytes are scaled by the same factors
    copy = 256 << 20
    hdr = "Kernel_Name,Grid_Size,Workgroup_Size,Counter_Name,Counter_Value"
    k = '"void mx::(anonymous namespace)::mxfp8_quantize_kernel<mx::QuantArgs, false>(mx::QuantArgs)"'
    fetch = [hdr, '"__amd_rocclr_copyBuffer",1024,256,FETCH_SIZE,%f' % (copy / 2 / 1024),
             "%s,262144,256,FETCH_SIZE,1000" % k]
    write = [hdr, '"__amd_rocclr_copyBuffer",1024,256,WRITE_SIZE,%f' % (copy / 1024),
             "%s,262144,256,WRITE_SIZE,3000" % k]
    (tmp_path / "f.csv").write_text("\n".join(fetch) + "\n")
    (tmp_path / "w.csv").write_text("\n".join(write) + "\n")
    res = bench.traffic_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    assert res["fetch_scale"] == pytest.approx(2.0) and res["write_scale"] == pytest.approx(1.0)
    (key, rec), = res["kernels"].items()
    assert key == "mx::mxfp8_quantize_kernel<mx::QuantArgs, false>/1024"
    assert rec["bytes_per_launch"] == pytest.approx(2000 * 1024 + 3000 * 1024)
    assert rec["sources_hash"] == bench.sources_hash(key)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr

"""The C ABI calls inside captured HIP graphs: several replays, with the
program's own eager work and synchronizations between them, each checked
against the eager result on the same inputs."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_02_amd as mx
from mxfp8_block_scaled_02_amd import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def host(t):
    return t.cpu().numpy()


def test_graph_replays_match_eager():
    print("[case] graph: quantize row+col [256, 1056], rmsnorm_quantize [64, 7168], dequantize",
          flush=True)
    x = synth.weight_with_outliers(256, 1056, seed=31).to(DEV)
    xn, gamma = synth.rmsnorm_inputs(64, 7168, seed=32, x_std=3.0, row_decades=2.0)
    xn, gamma = xn.to(DEV), gamma.to(DEV)
    planes = mx.quantize(x, True, True)
    normed, q, s = mx.rmsnorm_quantize(xn, gamma, 0.5, 1e-5)
    deq = mx.dequantize(planes.columnwise_data, planes.columnwise_scale, mx.COLUMNWISE)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mx.quantize(x, True, True, out=planes)
        mx.rmsnorm_quantize(xn, gamma, 0.5, 1e-5, out=(normed, q, s))
        mx.dequantize(planes.columnwise_data, planes.columnwise_scale, mx.COLUMNWISE, out=deq)
    for rep in range(4):
        # eager work between replays: new inputs, written in place
        x.copy_(synth.weight_with_outliers(256, 1056, seed=100 + rep).to(DEV))
        xn.mul_(1.5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = mx.quantize(x.clone(), True, True)
        wn, wq, ws = mx.rmsnorm_quantize(xn.clone(), gamma, 0.5, 1e-5)
        wd = mx.dequantize(want.columnwise_data, want.columnwise_scale, mx.COLUMNWISE)
        torch.cuda.synchronize()
        for a, b in zip(planes, want):
            assert np.array_equal(host(a), host(b)), "replay %d: quantize planes differ" % rep
        assert np.array_equal(host(normed.view(torch.int16)), host(wn.view(torch.int16)))
        assert np.array_equal(host(q), host(wq)) and np.array_equal(host(s), host(ws))
        assert np.array_equal(host(deq.view(torch.int32)), host(wd.view(torch.int32)))


def test_graph_replays_match_eager_f32_grouped_and_gemm():
    """float32 input, a grouped call and the activation quantize followed by
    the matrix product (skinny kernel, and ring tiles with a short last scale
    group), captured together; both products are deterministic, so every
    replay must equal the eager calls bit for bit."""
    print("[case] graph: quantize f32 [128, 512], grouped [64, 256] [96, 1024] [32, 544], "
          "quantize + gemm 40x300x1024 and 300x512x640", flush=True)
    xf = synth.weight_with_outliers(128, 512, seed=51).to(DEV).float()
    xs = [synth.weight_with_outliers(r, c, seed=52 + i).to(DEV)
          for i, (r, c) in enumerate([(64, 256), (96, 1024), (32, 544)])]
    a1 = synth.weight_with_outliers(40, 1024, seed=56).to(DEV)
    a2 = synth.weight_with_outliers(300, 640, seed=57).to(DEV)
    b1 = mx.quantize(synth.weight_with_outliers(300, 1024, seed=58).to(DEV), True, False)
    b2 = mx.quantize(synth.weight_with_outliers(512, 640, seed=59).to(DEV), True, False)
    pf = mx.quantize(xf, True, True)
    pg = mx.quantize_grouped(xs, True, True)
    pa1, pa2 = mx.quantize(a1, True, False), mx.quantize(a2, True, False)
    c1 = mx.gemm(pa1.rowwise_data, pa1.rowwise_scale, b1.rowwise_data, b1.rowwise_scale, torch.float32)
    c2 = mx.gemm(pa2.rowwise_data, pa2.rowwise_scale, b2.rowwise_data, b2.rowwise_scale, torch.bfloat16)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mx.quantize(xf, True, True, out=pf)
        mx.quantize_grouped(xs, True, True, outs=pg)
        mx.quantize(a1, True, False, out=pa1)
        mx.quantize(a2, True, False, out=pa2)
        mx.gemm(pa1.rowwise_data, pa1.rowwise_scale, b1.rowwise_data, b1.rowwise_scale, torch.float32, out=c1)
        mx.gemm(pa2.rowwise_data, pa2.rowwise_scale, b2.rowwise_data, b2.rowwise_scale, torch.bfloat16, out=c2)
    for rep in range(4):
        # eager work between replays: new inputs, written in place
        xf.mul_(-1.25)
        for x in xs:
            x.copy_((x.float() * 1.5).to(torch.bfloat16))
        a1.copy_(synth.weight_with_outliers(40, 1024, seed=200 + rep).to(DEV))
        a2.copy_(synth.weight_with_outliers(300, 640, seed=300 + rep).to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        wf = mx.quantize(xf.clone(), True, True)
        wg = mx.quantize_grouped([x.clone() for x in xs], True, True)
        w1, w2 = mx.quantize(a1.clone(), True, False), mx.quantize(a2.clone(), True, False)
        d1 = mx.gemm(w1.rowwise_data, w1.rowwise_scale, b1.rowwise_data, b1.rowwise_scale, torch.float32)
        d2 = mx.gemm(w2.rowwise_data, w2.rowwise_scale, b2.rowwise_data, b2.rowwise_scale, torch.bfloat16)
        torch.cuda.synchronize()
        for got, want in [(pf, wf)] + list(zip(pg, wg)) + [(pa1, w1), (pa2, w2)]:
            for a, b in zip(got, want):
                if a is not None or b is not None:
                    assert np.array_equal(host(a), host(b)), "replay %d: planes differ" % rep
        assert np.array_equal(host(c1.view(torch.int32)), host(d1.view(torch.int32))), "replay %d: skinny" % rep
        assert np.array_equal(host(c2.view(torch.int16)), host(d2.view(torch.int16))), "replay %d: ring" % rep


def test_graph_replays_match_eager_transposed_and_grouped_gemm():
    """The transposed columnwise plane (bf16 and float32 input) and a grouped
    product with skinny and ring-tile tables, captured together: every replay
    equals the eager calls bit for bit."""
    print("[case] graph: transposed quantize bf16 [256, 520] and f32 [160, 264], grouped gemm "
          "of 5 experts", flush=True)
    x = synth.weight_with_outliers(256, 520, seed=61).to(DEV)
    xf = synth.weight_with_outliers(160, 264, seed=62).to(DEV).float()
    toks, widths, K = [1, 20, 64, 200, 0], [256, 384, 512, 300, 128], 1024
    A = [synth.weight_with_outliers(m, K, seed=70 + i).to(DEV) for i, m in enumerate(toks)]
    W = [mx.quantize(synth.weight_with_outliers(n, K, seed=80 + i).to(DEV), True, False) for i, n in enumerate(widths)]
    pt = mx.quantize(x, False, True, columnwise_transposed=True)
    pft = mx.quantize(xf, False, True, columnwise_transposed=True)
    pa = [mx.quantize(a, True, False) for a in A]
    ys = mx.gemm_grouped([p.rowwise_data for p in pa], [p.rowwise_scale for p in pa],
                         [w.rowwise_data for w in W], [w.rowwise_scale for w in W], torch.bfloat16)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mx.quantize(x, False, True, out=pt, columnwise_transposed=True)
        mx.quantize(xf, False, True, out=pft, columnwise_transposed=True)
        for a, p in zip(A, pa):
            mx.quantize(a, True, False, out=p)
        mx.gemm_grouped([p.rowwise_data for p in pa], [p.rowwise_scale for p in pa],
                        [w.rowwise_data for w in W], [w.rowwise_scale for w in W], torch.bfloat16, outs=ys)
    for rep in range(4):
        x.copy_(synth.weight_with_outliers(256, 520, seed=400 + rep).to(DEV))
        xf.mul_(-0.75)
        for i, a in enumerate(A):
            a.copy_(synth.weight_with_outliers(toks[i], K, seed=500 + 10 * rep + i).to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        wt = mx.quantize(x.clone(), False, True, columnwise_transposed=True)
        wft = mx.quantize(xf.clone(), False, True, columnwise_transposed=True)
        wa = [mx.quantize(a.clone(), True, False) for a in A]
        wy = mx.gemm_grouped([p.rowwise_data for p in wa], [p.rowwise_scale for p in wa],
                             [w.rowwise_data for w in W], [w.rowwise_scale for w in W], torch.bfloat16)
        torch.cuda.synchronize()
        for got, want in ((pt, wt), (pft, wft)):
            assert np.array_equal(host(got.columnwise_data), host(want.columnwise_data)), "replay %d" % rep
            assert np.array_equal(host(got.columnwise_scale), host(want.columnwise_scale)), "replay %d" % rep
        for i, (y, w) in enumerate(zip(ys, wy)):
            assert np.array_equal(host(y.view(torch.int16)), host(w.view(torch.int16))), "replay %d expert %d" % (rep, i)


def test_calls_run_on_the_current_stream():
    """Every entry point launches on the caller's current stream: on a side
    stream held up by a long sleep, then given a new input, each result must
    reflect that new input (a launch on any other stream would read the old
    one)."""
    print("[case] side stream: quantize, quantize_f32, rmsnorm_quantize, dequantize, gemm", flush=True)
    x = synth.weight_with_outliers(256, 1056, seed=41).to(DEV)
    x_new = synth.weight_with_outliers(256, 1056, seed=42).to(DEV)
    xf = x.float()
    xf_new = x_new.float()
    xn, gamma = synth.rmsnorm_inputs(64, 7168, seed=43, x_std=3.0, row_decades=2.0)
    xn, gamma = xn.to(DEV), gamma.to(DEV)
    xn_new = (xn.float() * 3.0).to(torch.bfloat16)
    a = synth.weight_with_outliers(96, 512, seed=44).to(DEV)
    a_new = synth.weight_with_outliers(96, 512, seed=45).to(DEV)
    b = mx.quantize(synth.weight_with_outliers(160, 512, seed=46).to(DEV), True, False)
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=DEV)     # default priority
    with torch.cuda.stream(side):
        torch.cuda._sleep(20_000_000)        # hold the stream for several milliseconds
        x.copy_(x_new)
        xf.copy_(xf_new)
        xn.copy_(xn_new)
        a.copy_(a_new)
        p = mx.quantize(x, True, True)
        pf = mx.quantize(xf, True, True)
        normed, q, s = mx.rmsnorm_quantize(xn, gamma, 0.5, 1e-5)
        pa = mx.quantize(a, True, False)
        d = mx.dequantize(p.columnwise_data, p.columnwise_scale, mx.COLUMNWISE)
        out = mx.gemm(pa.rowwise_data, pa.rowwise_scale, b.rowwise_data, b.rowwise_scale)
    torch.cuda.synchronize()
    want = mx.quantize(x_new, True, True)
    wantf = mx.quantize(xf_new, True, True)
    wn, wq, ws = mx.rmsnorm_quantize(xn_new, gamma, 0.5, 1e-5)
    wa = mx.quantize(a_new, True, False)
    wd = mx.dequantize(want.columnwise_data, want.columnwise_scale, mx.COLUMNWISE)
    wo = mx.gemm(wa.rowwise_data, wa.rowwise_scale, b.rowwise_data, b.rowwise_scale)
    torch.cuda.synchronize()
    for got, exp in zip(list(p) + list(pf), list(want) + list(wantf)):
        assert np.array_equal(host(got), host(exp)), "quantize did not see the side stream's input"
    assert np.array_equal(host(normed.view(torch.int16)), host(wn.view(torch.int16)))
    assert np.array_equal(host(q), host(wq)) and np.array_equal(host(s), host(ws))
    assert np.array_equal(host(d.view(torch.int32)), host(wd.view(torch.int32)))
    assert np.array_equal(host(out.view(torch.int32)), host(wo.view(torch.int32)))

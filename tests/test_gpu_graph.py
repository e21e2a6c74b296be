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

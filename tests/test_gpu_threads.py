"""The library keeps no state: four host threads, each on a stream of its own
(default priority), call every entry point at once, many times over, and every
result equals the one computed beforehand on the main thread, bit for bit."""
import threading

import pytest
import torch

import mxfp8_block_scaled_02_amd as mx

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def bf16(rows, cols, seed, std=1.0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (torch.randn(rows, cols, generator=g, device=DEV) * std).to(torch.bfloat16)


def work(x, gamma, w):
    """Every entry point on one thread's inputs; outputs as a flat list."""
    p = mx.quantize(x, True, True)
    n, q, s = mx.rmsnorm_quantize(x, gamma, 0.5, 1e-5)
    d = mx.dequantize(p.columnwise_data, p.columnwise_scale, mx.COLUMNWISE, torch.float32)
    g = mx.quantize_grouped([x, w], True, True)
    y = mx.gemm(p.rowwise_data, p.rowwise_scale, g[1].rowwise_data, g[1].rowwise_scale, torch.bfloat16)
    t = mx.quantize(x, False, True, columnwise_transposed=True)
    yg = mx.gemm_grouped([p.rowwise_data[:16], p.rowwise_data], [p.rowwise_scale[:16], p.rowwise_scale],
                         [g[1].rowwise_data, g[1].rowwise_data], [g[1].rowwise_scale, g[1].rowwise_scale])
    return [p.rowwise_data, p.rowwise_scale, p.columnwise_data, p.columnwise_scale, n, q, s, d,
            g[0].columnwise_data, y, t.columnwise_data, t.columnwise_scale] + yg


def same(a, b):
    if a.dtype in (torch.float32, torch.bfloat16):
        a, b = a.view(torch.int32 if a.dtype == torch.float32 else torch.int16), \
            b.view(torch.int32 if b.dtype == torch.float32 else torch.int16)
    return torch.equal(a, b)


def test_concurrent_calls_on_separate_streams():
    inputs = [(bf16(256, 1024, 10 + i, 2.0), bf16(1, 1024, 20 + i).reshape(1024), bf16(512, 1024, 30 + i, 0.05))
              for i in range(4)]
    want = [work(*inp) for inp in inputs]
    torch.cuda.synchronize()
    errors = []

    def run(i):
        try:
            stream = torch.cuda.Stream(device=DEV)           # default priority
            with torch.cuda.stream(stream):
                for _ in range(25):
                    got = work(*inputs[i])
                    stream.synchronize()
                    if not all(same(a, b) for a, b in zip(got, want[i])):
                        errors.append("thread %d: a result differs" % i)
                        return
        except Exception as e:                                # surfaced below
            errors.append("thread %d: %r" % (i, e))

    print("[case] four threads, separate streams", flush=True)
    threads = [threading.Thread(target=run, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=100)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors

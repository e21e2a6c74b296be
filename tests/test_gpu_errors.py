"""Refused calls on the GPU: every argument is checked before the first launch,
so a grouped call with one bad tensor raises and leaves the outputs of its
valid tensors untouched (filled with 0xA5 beforehand); bad single calls raise
ValueError before touching the GPU."""
import pytest
import torch

import mxfp8_block_scaled_02_amd as mx

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
FILL = 0xA5


def filled(shape, dtype=torch.uint8):
    t = torch.empty(shape, dtype=dtype, device=DEV)
    t.view(torch.uint8).fill_(FILL)
    return t


def untouched(*ts):
    torch.cuda.synchronize()
    return all(bool((t.view(torch.uint8) == FILL).all()) for t in ts)


def bf16(rows, cols, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return torch.randn(rows, cols, generator=g, device=DEV).to(torch.bfloat16)


def test_grouped_quantize_refused_writes_nothing():
    good = bf16(64, 512, 1)
    bad = bf16(64, 40, 2)                      # 40 columns: no whole rowwise blocks
    o = mx.MXFP8Planes(filled((64, 512)), filled((64, 512)), filled((64, 16)), filled((2, 512)))
    print("[case] grouped quantize with a partial block", flush=True)
    with pytest.raises(ValueError):
        mx.quantize_grouped([good, bad], True, True, outs=[o, None])
    assert untouched(*o)


def test_grouped_rmsnorm_refused_writes_nothing():
    xs = [bf16(8, 1024, 3), bf16(8, 1024, 4)]
    gs = [torch.ones(1024, dtype=torch.bfloat16, device=DEV)] * 2
    outs = [(filled((8, 1024), torch.bfloat16), filled((8, 1024)), filled((8, 32))), None]
    print("[case] grouped rmsnorm with a negative eps", flush=True)
    with pytest.raises(ValueError):
        mx.rmsnorm_quantize_grouped(xs, gs, [0.0, 0.0], [1e-6, -1.0], outs=outs)
    assert untouched(*outs[0])


def test_grouped_dequantize_refused_writes_nothing():
    p = mx.quantize(bf16(64, 512, 5), True, True)
    q_bad = torch.zeros((40, 512), dtype=torch.uint8, device=DEV)     # 40 rows: no whole column blocks
    s_bad = torch.zeros((1, 512), dtype=torch.uint8, device=DEV)
    out = filled((64, 512), torch.float32)
    print("[case] grouped dequantize with a partial column block", flush=True)
    with pytest.raises(ValueError):
        mx.dequantize_grouped([p.rowwise_data, q_bad], [p.rowwise_scale, s_bad], [mx.ROWWISE, mx.COLUMNWISE],
                              torch.float32, outs=[out, None])
    assert untouched(out)


def test_single_calls_refused():
    x = bf16(64, 512, 6)
    print("[case] single calls with bad arguments", flush=True)
    with pytest.raises(ValueError, match="contiguous"):
        mx.quantize(x.t(), True, False)
    with pytest.raises(ValueError):
        mx.quantize(x.to(torch.float16), True, False)
    with pytest.raises(ValueError):
        mx.quantize(bf16(40, 512, 7), False, True)                   # 40 rows, columnwise
    with pytest.raises(ValueError):
        mx.quantize(bf16(64, 96, 8), True, False, scale_order="mfma")   # the MFMA order needs cols % 512
    with pytest.raises(ValueError):
        mx.rmsnorm_quantize(x, torch.ones(256, dtype=torch.bfloat16, device=DEV))
    p = mx.quantize(x, True, False)
    with pytest.raises(ValueError):
        mx.dequantize(p.rowwise_data, p.rowwise_scale[:, :8], mx.ROWWISE)
    w = mx.quantize(bf16(128, 256, 9), True, False)
    with pytest.raises(ValueError):
        mx.gemm(p.rowwise_data, p.rowwise_scale, w.rowwise_data, w.rowwise_scale)   # K 512 vs 256
    torch.cuda.synchronize()

"""Refused calls on the GPU: every argument is checked before the first launch,
so a grouped call with one bad tensor or product raises and leaves the
outputs of its valid ones untouched (filled with 0xA5 beforehand); bad single
calls raise ValueError before touching the GPU."""
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


def test_grouped_gemm_refused_writes_nothing():
    """A grouped product whose last descriptor is bad (K not a multiple of
    128) raises before any launch: the valid products' outputs (skinny and
    ring-tile tables) keep their 0xA5 fill."""
    def quantized(rows, K, seed):
        p = mx.quantize(bf16(rows, K, seed), True, False)
        return p.rowwise_data, p.rowwise_scale
    qa, sa = zip(*[quantized(m, 512, 10 + i) for i, m in enumerate((8, 200))])
    qb, sb = zip(*[quantized(n, 512, 20 + i) for i, n in enumerate((256, 384))])
    outs = [filled((8, 256), torch.float32), filled((200, 384), torch.float32)]
    G = mx._GemmDesc
    descs = [G(qa[i].data_ptr(), sa[i].data_ptr(), qb[i].data_ptr(), sb[i].data_ptr(), qa[i].shape[0],
               qb[i].shape[0], 512, 0, 0, outs[i].data_ptr(), 0) for i in range(2)]
    descs.append(G(qa[0].data_ptr(), sa[0].data_ptr(), qb[0].data_ptr(), sb[0].data_ptr(), 8, 256, 96, 0, 0,
                   outs[0].data_ptr(), 0))
    print("[case] grouped gemm with a bad last product", flush=True)
    status = mx.lib().mxfp8_gemm_grouped((G * 3)(*descs), 3, 0, mx._stream(DEV))
    assert status == 2                                     # MXFP8_ERR_SHAPE
    assert untouched(*outs)


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

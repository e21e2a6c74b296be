"""Scale planes inside padded allocations (rows a pitch apart): every entry
point writes or reads them in place, the valid region equals the compact
result byte for byte, and the padding is never touched.

The pages name a padded consumer allocation (quantized_dbuffer page,
_pad_rowwise_scale / _pad_columnwise_scale) without giving its shape; the
padding multiples used here (rows to 128 and 4, columns to 4 and 128) are
examples of such a shape, not a claim about any other library's layout.
"""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_02_amd as mx
from mxfp8_block_scaled_02_amd import synth
from tests import gemm_accuracy as acc

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
FILL = 0xA5


def say(*a):
    print("[case]", *a, flush=True)


def padded(rows, cols, axis, rm, cm):
    return mx.padded_scale_plane(rows, cols, axis, rm, cm, device=DEV, fill=FILL)


def untouched(buf, view):
    """Every byte of buf outside view still holds FILL."""
    mask = torch.ones_like(buf, dtype=torch.bool)
    mask[:view.shape[0], :view.shape[1]] = False
    return bool((buf[mask] == FILL).all())


def bf16_input(rows, cols, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(rows, cols, generator=g) * 0.5).to(torch.bfloat16).to(DEV)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape,columnwise", [((100, 1056), False), ((96, 1056), True),
                                              ((1, 64), False), ((2048, 512), True),
                                              # more tiles than are resident at once (scale
                                              # bytes written back rather than streamed)
                                              ((4096, 8192), True)])
def test_quantize_into_padded_scales(shape, columnwise, dtype):
    rows, cols = shape
    say("quantize padded", shape, "col" if columnwise else "row", dtype)
    x = bf16_input(rows, cols, seed=rows + cols).to(dtype)
    ref = mx.quantize(x, True, columnwise)
    rbuf, rview = padded(rows, cols, mx.ROWWISE, 128, 4)
    cbuf = cview = None
    if columnwise:
        cbuf, cview = padded(rows, cols, mx.COLUMNWISE, 4, 128)
    got = mx.quantize(x, True, columnwise, out=mx.MXFP8Planes(None, None, rview, cview))
    torch.cuda.synchronize()
    assert torch.equal(got.rowwise_data, ref.rowwise_data)
    assert torch.equal(rview, ref.rowwise_scale) and untouched(rbuf, rview)
    if columnwise:
        assert torch.equal(got.columnwise_data, ref.columnwise_data)
        assert torch.equal(cview, ref.columnwise_scale) and untouched(cbuf, cview)


@pytest.mark.parametrize("rows,cols", [(37, 7168), (16, 1024), (300, 64)])
def test_rmsnorm_into_padded_scales(rows, cols):
    say("rmsnorm padded", rows, cols)
    x, gamma = synth.rmsnorm_inputs(rows, cols, seed=rows, device=DEV)
    normed, q, s = mx.rmsnorm_quantize(x, gamma, 0.5, 1e-5)
    buf, view = padded(rows, cols, mx.ROWWISE, 128, 4)
    n2, q2, s2 = mx.rmsnorm_quantize(x, gamma, 0.5, 1e-5, out=(None, None, view))
    torch.cuda.synchronize()
    assert torch.equal(n2, normed) and torch.equal(q2, q)
    assert torch.equal(view, s) and untouched(buf, view)


def test_grouped_mixed_padded_and_compact():
    """40 tensors, every other one with padded scales: more than one pitched
    launch, and each result equal to its single compact call."""
    g = torch.Generator().manual_seed(7)
    xs, outs, bufs = [], [], []
    for i in range(40):
        rows = 32 * int(torch.randint(1, 5, (1,), generator=g))
        cols = 32 * int(torch.randint(1, 40, (1,), generator=g))
        xs.append(bf16_input(rows, cols, seed=100 + i))
        if i % 2:
            rb, rv = padded(rows, cols, mx.ROWWISE, 64, 8)
            cb, cv = padded(rows, cols, mx.COLUMNWISE, 2, 64)
            outs.append(mx.MXFP8Planes(None, None, rv, cv))
            bufs.append((rb, rv, cb, cv))
        else:
            outs.append(None)
            bufs.append(None)
    say("grouped mixed padded", len(xs))
    got = mx.quantize_grouped(xs, True, True, outs=outs)
    for i, x in enumerate(xs):
        ref = mx.quantize(x, True, True)
        p = got[i]
        assert torch.equal(p.rowwise_data, ref.rowwise_data) and torch.equal(p.columnwise_data, ref.columnwise_data)
        assert torch.equal(p.rowwise_scale, ref.rowwise_scale)
        assert torch.equal(p.columnwise_scale, ref.columnwise_scale)
        if bufs[i]:
            rb, rv, cb, cv = bufs[i]
            assert untouched(rb, rv) and untouched(cb, cv)


@pytest.mark.parametrize("axis", [mx.ROWWISE, mx.COLUMNWISE])
def test_dequantize_from_padded_scales(axis):
    rows, cols = 160, 2080
    say("dequantize padded", axis)
    x = bf16_input(rows, cols, seed=3)
    planes = mx.quantize(x, True, True)
    q = planes.rowwise_data if axis == mx.ROWWISE else planes.columnwise_data
    s = planes.rowwise_scale if axis == mx.ROWWISE else planes.columnwise_scale
    buf, view = padded(rows, cols, axis, 8, 8 if axis == mx.ROWWISE else 128)
    view.copy_(s)
    for dt in (torch.float32, torch.bfloat16):
        a = mx.dequantize(q, s, axis, dt)
        b = mx.dequantize(q, view, axis, dt)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32 if dt == torch.float32 else torch.int16),
                           b.view(torch.int32 if dt == torch.float32 else torch.int16))


@pytest.mark.parametrize("mnk,pitch_multiple", [((4096, 4096, 512), 32), ((16, 2048, 1024), 36),
                                                ((300, 500, 384), 16),
                                                # four A tiles: staged scale words, then paired
                                                ((100, 1000, 1024), 20), ((96, 300, 16896), 36)])
def test_gemm_reads_padded_scales(mnk, pitch_multiple):
    """The same kernel runs for compact and padded planes here, so the outputs
    agree bit for bit; the planes come from quantizing into padded buffers."""
    M, N, K = mnk
    say("gemm padded", mnk, pitch_multiple)
    a = bf16_input(M, K, seed=M)
    b = (bf16_input(N, K, seed=N) * 0.05).to(torch.bfloat16)
    pa, pb = mx.quantize(a, True, False), mx.quantize(b, True, False)
    _, sav = padded(M, K, mx.ROWWISE, 1, pitch_multiple)
    _, sbv = padded(N, K, mx.ROWWISE, 1, pitch_multiple)
    qa2 = mx.quantize(a, True, False, out=mx.MXFP8Planes(None, None, sav, None)).rowwise_data
    qb2 = mx.quantize(b, True, False, out=mx.MXFP8Planes(None, None, sbv, None)).rowwise_data
    ref = mx.gemm(pa.rowwise_data, pa.rowwise_scale, pb.rowwise_data, pb.rowwise_scale, torch.float32)
    got = mx.gemm(qa2, sav, qb2, sbv, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))


@pytest.mark.parametrize("mnk,pitch", [((4096, 4096, 512), 20), ((4100, 1000, 640), 24),
                                       ((300, 2000, 1152), 40)])
def test_gemm_padded_scales_large(orc, mnk, pitch):
    """A pitch that is a multiple of 4 but not of 16 puts the ring tiles' 16-byte
    scale loads at 4-byte aligned addresses, also where K % 512 != 0 shifts the
    last group's load back: checked against the oracle at sampled positions."""
    M, N, K = mnk
    say("gemm padded", mnk, "pitch", pitch)
    a = bf16_input(M, K, seed=11)
    b = (bf16_input(N, K, seed=12) * 0.05).to(torch.bfloat16)
    pa, pb = mx.quantize(a, True, False), mx.quantize(b, True, False)
    _, sav = padded(M, K, mx.ROWWISE, 1, pitch)
    _, sbv = padded(N, K, mx.ROWWISE, 1, pitch)
    sav.copy_(pa.rowwise_scale)
    sbv.copy_(pb.rowwise_scale)
    got = mx.gemm(pa.rowwise_data, sav, pb.rowwise_data, sbv, torch.float32)
    torch.cuda.synchronize()
    g = np.random.default_rng(5)
    ms, ns = g.integers(0, M, 3000), g.integers(0, N, 3000)
    host = lambda t: t.cpu().numpy()
    planes = [host(pa.rowwise_data), host(pa.rowwise_scale), host(pb.rowwise_data), host(pb.rowwise_scale)]
    C, _ = orc.gemm_at(*planes, ms, ns)
    err = np.abs(host(got)[ms, ns].astype(np.float64) - C)
    assert (err <= acc.bound_at(*planes, ms, ns)).all()


def test_scale_view_strides_checked():
    """A one-row scale view whose columns are not adjacent bytes is refused
    (the library writes each scale row as consecutive bytes)."""
    say("scale view strides")
    buf = torch.zeros((32, 64), dtype=torch.uint8, device=DEV)
    bad = buf[:1, ::2]                                    # [1, 32], column stride 2
    assert bad.shape == (1, 32) and bad.stride(1) == 2
    with pytest.raises(ValueError, match="unit column stride"):
        # columnwise scales of a [32, 32] tensor are [1, 32]
        mx.quantize(bf16_input(32, 32, seed=21), False, True, out=mx.MXFP8Planes(None, None, None, bad))
    with pytest.raises(ValueError, match="unit column stride"):
        # rowwise scales of a [1, 1024] tensor are [1, 32]
        mx.quantize(bf16_input(1, 1024, seed=21), True, False, out=mx.MXFP8Planes(None, None, bad, None))
    assert bool((buf == 0).all())


def test_float8_views_accepted():
    """Planes viewed with the float8 dtypes (as_fp8) are accepted wherever
    byte planes are, and give the same results."""
    say("float8 views")
    x = bf16_input(256, 512, seed=22)
    w = (bf16_input(384, 512, seed=23) * 0.05).to(torch.bfloat16)
    pa, pb = mx.quantize(x, True, True), mx.quantize(w, True, False)
    fa, fb = mx.as_fp8(pa), mx.as_fp8(pb)
    ref = mx.gemm(pa.rowwise_data, pa.rowwise_scale, pb.rowwise_data, pb.rowwise_scale)
    got = mx.gemm(fa.rowwise_data, fa.rowwise_scale, fb.rowwise_data, fb.rowwise_scale)
    d_ref = mx.dequantize(pa.columnwise_data, pa.columnwise_scale, mx.COLUMNWISE)
    d_got = mx.dequantize(fa.columnwise_data, fa.columnwise_scale, mx.COLUMNWISE)
    outs = mx.as_fp8(mx.MXFP8Planes(*(torch.empty_like(t) for t in pa)))
    again = mx.quantize(x, True, True, out=outs)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))
    assert torch.equal(d_got.view(torch.int32), d_ref.view(torch.int32))
    for a, b in zip(again, pa):
        assert torch.equal(a, b)
    assert torch.equal(outs.rowwise_data.view(torch.uint8), pa.rowwise_data)

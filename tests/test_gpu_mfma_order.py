"""Rowwise scales in the MFMA order (include/mxfp8.h, "Scale pitches"): every
kernel that writes or reads rowwise scales, against the same call with compact
scales.  The expected plane is the compact one permuted by the order's
definition, block b of row r at [b // 16, r, b % 16]; the compact planes
themselves are checked against the oracle by the other GPU tests, and here
once more on the small cases."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_02_amd as mx
from mxfp8_block_scaled_02_amd import synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
GUARD = 0xA5


def say(*a):
    print("[case]", *a, flush=True)


def to_mfma(compact):
    """[rows, cols/32] -> [cols/512, rows, 16] by the definition."""
    c = np.asarray(compact)
    rows, w = c.shape
    return c.reshape(rows, w // 16, 16).transpose(1, 0, 2)


def guarded_mfma(rows, cols, pad=4096):
    """A plane in the MFMA order inside a buffer filled with GUARD: (buffer,
    plane view)."""
    n = rows * cols // 32
    buf = torch.full((pad + n + pad,), GUARD, dtype=torch.uint8, device=DEV)
    return buf, buf[pad:pad + n].view(mx.mfma_scale_shape(rows, cols))


def assert_guards(buf, n, pad=4096):
    b = buf.cpu().numpy()
    assert (b[:pad] == GUARD).all() and (b[pad + n:] == GUARD).all(), "write outside the plane"


def bf16(rows, cols, seed, std=1.0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (torch.randn(rows, cols, generator=g, device=DEV) * std).to(torch.bfloat16)


@pytest.mark.parametrize("shape", [(32, 512), (64, 1024), (4096, 4096), (8192, 4096), (96, 7168)])
@pytest.mark.parametrize("columnwise", [True, False])
def test_quantize_bf16(orc, shape, columnwise):
    """Row + column tiles (resident and streaming grids) and the flat rowwise
    path (one piece a lane for small tensors, four for large)."""
    rows, cols = shape
    say("quantize bf16 mfma", shape, columnwise)
    x = bf16(rows, cols, rows + cols)
    ref = mx.quantize(x, True, columnwise)
    buf, plane = guarded_mfma(rows, cols)
    out = mx.MXFP8Planes(None, None, plane, None)
    got = mx.quantize(x, True, columnwise, out=out, scale_order="mfma")
    torch.cuda.synchronize()
    assert got.rowwise_scale.data_ptr() == plane.data_ptr()
    assert np.array_equal(got.rowwise_scale.cpu().numpy(), to_mfma(ref.rowwise_scale.cpu().numpy()))
    assert torch.equal(got.rowwise_data, ref.rowwise_data)
    if columnwise:
        assert torch.equal(got.columnwise_data, ref.columnwise_data)
        assert torch.equal(got.columnwise_scale, ref.columnwise_scale)
    assert_guards(buf, rows * cols // 32)
    if rows * cols <= 1 << 16:
        _, s = orc.quantize_rowwise(synth.bf16_bits(x.cpu()))
        assert np.array_equal(got.rowwise_scale.cpu().numpy(), to_mfma(s))


@pytest.mark.parametrize("shape", [(32, 512), (4096, 4096), (256, 1024)])
@pytest.mark.parametrize("columnwise", [True, False])
def test_quantize_f32(shape, columnwise):
    rows, cols = shape
    say("quantize f32 mfma", shape, columnwise)
    g = torch.Generator(device=DEV).manual_seed(7)
    x = torch.randn(rows, cols, generator=g, device=DEV) * 0.02
    ref = mx.quantize(x, True, columnwise)
    got = mx.quantize(x, True, columnwise, scale_order="mfma")
    torch.cuda.synchronize()
    assert np.array_equal(got.rowwise_scale.cpu().numpy(), to_mfma(ref.rowwise_scale.cpu().numpy()))
    assert torch.equal(got.rowwise_data, ref.rowwise_data)


def test_quantize_grouped_mixed_orders():
    """One grouped launch with compact, padded and MFMA-order planes: the
    pitched instantiation serves all three."""
    xs = [bf16(64, 1024, 1), bf16(96, 512, 2), bf16(32, 1536, 3)]
    say("quantize grouped mixed orders")
    refs = mx.quantize_grouped(xs, True, True)
    _, padded = mx.padded_scale_plane(96, 512, mx.ROWWISE, 1, 32, device=DEV, fill=GUARD)
    outs = [mx.MXFP8Planes(None, None, torch.empty(mx.mfma_scale_shape(64, 1024), dtype=torch.uint8,
                                                   device=DEV), None),
            mx.MXFP8Planes(None, None, padded, None),
            mx.MXFP8Planes(None, None, torch.empty(mx.mfma_scale_shape(32, 1536), dtype=torch.uint8,
                                                   device=DEV), None)]
    got = mx.quantize_grouped(xs, True, True, outs=outs)
    torch.cuda.synchronize()
    assert np.array_equal(got[0].rowwise_scale.cpu().numpy(), to_mfma(refs[0].rowwise_scale.cpu().numpy()))
    assert torch.equal(got[1].rowwise_scale, refs[1].rowwise_scale)
    assert np.array_equal(got[2].rowwise_scale.cpu().numpy(), to_mfma(refs[2].rowwise_scale.cpu().numpy()))
    for a, b in zip(got, refs):
        assert torch.equal(a.rowwise_data, b.rowwise_data) and torch.equal(a.columnwise_scale, b.columnwise_scale)


@pytest.mark.parametrize("shape", [(16, 7168), (300, 1024), (2048, 8192), (8, 16384), (4, 20480)])
def test_rmsnorm_quantize(shape):
    """Every RMSNorm variant: a wave per row, a workgroup per row, 16 waves per
    row for small launches, and rows read twice (over 16384 elements)."""
    rows, cols = shape
    say("rmsnorm mfma", shape)
    x = bf16(rows, cols, 11, 3.0)
    gamma = bf16(1, cols, 12).reshape(cols)
    rn, rq, rs = mx.rmsnorm_quantize(x, gamma, 1.0, 1e-5)
    buf, plane = guarded_mfma(rows, cols)
    n, q, s = mx.rmsnorm_quantize(x, gamma, 1.0, 1e-5, out=(None, None, plane))
    torch.cuda.synchronize()
    assert torch.equal(n, rn) and torch.equal(q, rq)
    assert np.array_equal(s.cpu().numpy(), to_mfma(rs.cpu().numpy()))
    assert_guards(buf, rows * cols // 32)


def test_rmsnorm_quantize_grouped_scale_order():
    xs = [bf16(8, 1024, 21), bf16(40, 2048, 22)]
    gs = [bf16(1, 1024, 23).reshape(-1), bf16(1, 2048, 24).reshape(-1)]
    say("rmsnorm grouped mfma")
    ref = mx.rmsnorm_quantize_grouped(xs, gs, [0.0, 1.0], [1e-6, 1e-5])
    got = mx.rmsnorm_quantize_grouped(xs, gs, [0.0, 1.0], [1e-6, 1e-5], scale_order="mfma")
    torch.cuda.synchronize()
    for (n, q, s), (rn, rq, rs) in zip(got, ref):
        assert torch.equal(n, rn) and torch.equal(q, rq)
        assert np.array_equal(s.cpu().numpy(), to_mfma(rs.cpu().numpy()))


@pytest.mark.parametrize("shape", [(32, 512), (4096, 4096), (100, 1536)])
def test_dequantize(shape):
    rows, cols = shape
    say("dequantize mfma", shape)
    x = bf16(rows, cols, 31)
    p = mx.quantize(x, True, False)
    pm = mx.quantize(x, True, False, scale_order="mfma")
    for dt in (torch.float32, torch.bfloat16):
        a = mx.dequantize(p.rowwise_data, p.rowwise_scale, mx.ROWWISE, dt)
        b = mx.dequantize(pm.rowwise_data, pm.rowwise_scale, mx.ROWWISE, dt)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


@pytest.mark.parametrize("mnk", [
    (1024, 1024, 512), (1024, 7168, 7168), (4352, 3840, 1536), (600, 2048, 4096),  # ring tiles
    (64, 18432, 1024), (100, 20480, 512),             # ring tiles under 33 .. 128 rows (a wide weight)
    (16, 4096, 4096), (40, 1000, 2048), (100, 200, 512), (300, 2048, 4096),       # skinny, staged words
    (16, 96, 16896), (40, 130, 16896), (100, 64, 8704),                           # skinny, paired words
    (1024, 512, 1024), (300, 2048, 8704)])            # skinny row blocks: 64 rows; 128 rows, paired words
def test_gemm_matches_compact_scales(mnk):
    """The product from MFMA-order scale planes equals the product from the
    compact planes bit for bit (same kernel, same order of accumulation), for
    A, B or both in the MFMA order.  With K = 16896 and 8704 the paired scale
    words' wave ranges start in the middle of a 16-block group (unit 66, 34 or
    50: 2 mod 4)."""
    M, N, K = mnk
    a = mx.quantize(bf16(M, K, M + K), True, False)
    b = mx.quantize(bf16(N, K, N + K, 0.05), True, False)
    am = mx.quantize(bf16(M, K, M + K), True, False, scale_order="mfma")
    bm = mx.quantize(bf16(N, K, N + K, 0.05), True, False, scale_order="mfma")
    for dt in (torch.float32, torch.bfloat16):
        say("gemm mfma", mnk, dt)
        ref = mx.gemm(a.rowwise_data, a.rowwise_scale, b.rowwise_data, b.rowwise_scale, dt)
        for sa, sb in ((am.rowwise_scale, b.rowwise_scale), (a.rowwise_scale, bm.rowwise_scale),
                       (am.rowwise_scale, bm.rowwise_scale)):
            got = mx.gemm(a.rowwise_data, sa, b.rowwise_data, sb, dt)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int32 if dt == torch.float32 else torch.int16),
                               ref.view(torch.int32 if dt == torch.float32 else torch.int16)), mnk


def test_gemm_mfma_order_against_oracle(orc):
    """One product from MFMA-order planes against the oracle's float64 sum of
    the compact planes, within the accumulation bound."""
    from tests import gemm_accuracy as acc
    M, N, K = 200, 300, 1024
    say("gemm mfma vs oracle", (M, N, K))
    a = mx.quantize(bf16(M, K, 41), True, False, scale_order="mfma")
    b = mx.quantize(bf16(N, K, 42, 0.05), True, False, scale_order="mfma")
    got = mx.gemm(a.rowwise_data, a.rowwise_scale, b.rowwise_data, b.rowwise_scale).cpu().numpy()
    # the compact planes, from the MFMA order by the definition
    sa = a.rowwise_scale.cpu().numpy().transpose(1, 0, 2).reshape(M, K // 32)
    sb = b.rowwise_scale.cpu().numpy().transpose(1, 0, 2).reshape(N, K // 32)
    qa, qb = a.rowwise_data.cpu().numpy(), b.rowwise_data.cpu().numpy()
    C, _ = orc.gemm(qa, sa, qb, sb)
    tol = acc.bound(qa, sa, qb, sb)
    assert (np.abs(got.astype(np.float64) - C) <= tol).all()

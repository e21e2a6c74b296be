"""GPU parity of the transposed columnwise plane (columnwise scale pitch
MXFP8_COLUMNWISE_T): its bytes equal the oracle's columnwise plane transposed,
the rowwise plane of the same launch equals the oracle's in every scale
layout, grouped lists may mix the layouts, nothing outside the planes is
written, and the planes serve as operands of the matrix product for the two
backward products (input gradient and weight gradient), checked against the
float64 product of the untransposed planes."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_02_amd as mx
from mxfp8_block_scaled_02_amd import synth
from tests import gemm_accuracy as acc
from tests.test_gpu_parity import DEV, assert_same, dev_bits, dev_f32, f32_specials, host, say, special_values

pytestmark = pytest.mark.gpu

# whole and partial 128 x 128 tiles: rows 32 .. 96 past a multiple of 128
# (waves past the end), columns 8 .. 120 past one (lanes past the end)
SHAPES = [(32, 8), (32, 32), (32, 128), (128, 128), (96, 520), (96, 544), (160, 136), (160, 160),
          (256, 1024), (64, 4104), (1024, 96), (352, 1184), (4096 + 32, 264)]


def mfma_to_compact(s, rows, cols):
    """Rowwise scales in the MFMA order [cols/512, rows, 16] -> [rows, cols/32]."""
    return s.reshape(cols // 512, rows, 16).transpose(1, 0, 2).reshape(rows, cols // 32)


def check(orc, bits, rowwise, what, scale_order="row", out=None):
    """bits: bf16 bit patterns (uint16) or float32 values."""
    say("transposed columnwise", what, bits.shape, bits.dtype, "row" if rowwise else "", scale_order)
    x = dev_bits(bits) if bits.dtype == np.uint16 else dev_f32(bits)
    p = mx.quantize(x, rowwise, True, out=out, scale_order=scale_order, columnwise_transposed=True)
    torch.cuda.synchronize()
    rows, cols = bits.shape
    qt, st = orc.quantize_colwise_t(bits)
    assert tuple(p.columnwise_data.shape) == (cols, rows)
    assert_same(host(p.columnwise_data), qt, what + " q_colT")
    assert_same(host(p.columnwise_scale), st, what + " s_colT")
    if rowwise:
        qr, sr = orc.quantize_rowwise(bits)
        assert_same(host(p.rowwise_data), qr, what + " q_row")
        s = host(p.rowwise_scale)
        assert_same(mfma_to_compact(s, rows, cols) if scale_order == "mfma" else s, sr, what + " s_row")
    return p


@pytest.mark.parametrize("shape", SHAPES)
def test_transposed_columnwise(orc, shape):
    rows, cols = shape
    bits = special_values(rows, cols, seed=rows + 7 * cols)
    check(orc, bits, False, "columnwise only")
    if cols % 32 == 0:
        check(orc, bits, True, "rowwise + columnwise")


def test_weight_4096_full(orc):
    """The 4096 x 4096 weight with outlier rows and columns, both planes."""
    bits = synth.bf16_bits(synth.weight_with_outliers())
    check(orc, bits, True, "weight 4096^2")


def test_rowwise_scale_layouts(orc):
    """The rowwise plane of the same launch in the MFMA order and in a padded
    allocation (guard bytes untouched)."""
    rows, cols = 256, 1536
    bits = special_values(rows, cols, seed=5)
    check(orc, bits, True, "mfma rowwise scales", scale_order="mfma")
    buf, view = mx.padded_scale_plane(rows, cols, mx.ROWWISE, row_multiple=128, col_multiple=64, device=DEV,
                                      fill=0xA5)
    p = check(orc, bits, True, "padded rowwise scales", out=mx.MXFP8Planes(None, None, view, None))
    assert p.rowwise_scale.data_ptr() == view.data_ptr()
    b = host(buf)
    mask = np.ones(b.shape, bool)
    mask[:rows, :cols // 32] = False
    assert (b[mask] == 0xA5).all(), "padding written"


def test_guard_bands(orc):
    """Planes inside larger buffers filled with 0xA5 / 0x5A: no byte outside
    the planes changes (partial tiles in both directions)."""
    rows, cols = 160, 392
    bits = special_values(rows, cols, seed=9)
    pad = 4096
    qbuf = torch.full((cols * rows + 2 * pad,), 0xA5, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((cols * rows // 32 + 2 * pad,), 0x5A, dtype=torch.uint8, device=DEV)
    out = mx.MXFP8Planes(None, qbuf[pad:pad + cols * rows].view(cols, rows), None,
                         sbuf[pad:pad + cols * rows // 32].view(cols, rows // 32))
    check(orc, bits, False, "guard bands", out=out)
    for b, fill in ((host(qbuf), 0xA5), (host(sbuf), 0x5A)):
        assert (b[:pad] == fill).all() and (b[-pad:] == fill).all(), "write outside the plane"


def test_grouped_mixed_layouts(orc):
    """One grouped call over tensors whose columnwise planes are stored
    transposed, untransposed, or not requested: every plane equals the
    oracle's (two launch sequences, one per layout)."""
    shapes = [(32, 32), (96, 544), (128, 7168), (160, 136), (64, 1024), (256, 96)]
    g = torch.Generator().manual_seed(33)
    xs = [(torch.randn(s, generator=g) * 10 ** (i - 3)).to(torch.bfloat16) for i, s in enumerate(shapes)]
    layouts = [True, False, True, True, False, True]
    rowwise = [True, True, True, False, True, True]
    devx = [x.to(DEV) for x in xs]            # alive until the launch is done
    descs, planes = [], []
    for x, t, r in zip(devx, layouts, rowwise):
        d, p = mx._quant_desc(x, r, True, None, False, t)
        descs.append(d)
        planes.append(p)
    say("grouped mixed layouts", shapes)
    arr = (mx._QuantDesc * len(descs))(*descs)
    mx._check(mx.lib().mxfp8_quantize_grouped(arr, len(descs), mx._stream(DEV)))
    torch.cuda.synchronize()
    for x, t, r, p in zip(xs, layouts, rowwise, planes):
        bits = synth.bf16_bits(x)
        qc, sc = orc.quantize_colwise_t(bits) if t else orc.quantize_colwise(bits)
        assert_same(host(p.columnwise_data), qc, "grouped q_col %s %s" % (tuple(x.shape), t))
        assert_same(host(p.columnwise_scale), sc, "grouped s_col %s %s" % (tuple(x.shape), t))
        if r:
            qr, sr = orc.quantize_rowwise(bits)
            assert_same(host(p.rowwise_data), qr, "grouped q_row")
            assert_same(host(p.rowwise_scale), sr, "grouped s_row")


def test_grouped_experts_equal_single_calls():
    """Eight expert weights [2048, 7168] in one grouped call, both planes,
    equal to single calls byte for byte."""
    ws = synth.expert_weights(n=8, device=DEV)
    say("grouped experts transposed", len(ws))
    got = mx.quantize_grouped(ws, True, True, columnwise_transposed=True)
    for w, p in zip(ws, got):
        single = mx.quantize(w, True, True, columnwise_transposed=True)
        torch.cuda.synchronize()
        for a, b in zip(p, single):
            assert torch.equal(a, b)


# float32 input: 128 x 128 tiles, so columns 8 .. 120 past a multiple of 128
F32_SHAPES = [(32, 8), (32, 32), (128, 128), (96, 136), (160, 264), (256, 1024), (1024, 40), (352, 1184)]


@pytest.mark.parametrize("shape", F32_SHAPES)
def test_transposed_columnwise_f32(orc, shape):
    """float32 input with specials (NaN, Inf, subnormals, the largest
    finite values) spread over 60 binades."""
    rows, cols = shape
    x = f32_specials(rows, cols, seed=rows + 3 * cols)
    check(orc, x, False, "f32 columnwise only")
    if cols % 32 == 0:
        check(orc, x, True, "f32 rowwise + columnwise")


def test_f32_master_weight_4096(orc):
    """The 4096 x 4096 float32 master weight (outliers, zero and subnormal
    tiles), both planes, and its rowwise scales in the MFMA order."""
    x = synth.master_weight_f32().numpy()
    check(orc, x, True, "f32 master weight")
    check(orc, x, True, "f32 master weight, mfma rowwise scales", scale_order="mfma")


def test_f32_grouped_equals_single_calls():
    g = torch.Generator().manual_seed(44)
    xs = [(torch.randn(s, generator=g) * 0.02).to(DEV) for s in ((256, 7168), (96, 520), (2048, 64), (32, 8))]
    say("f32 grouped transposed", [tuple(x.shape) for x in xs])
    for rw in (True, False):
        use = [x for x in xs if not rw or x.shape[1] % 32 == 0]
        got = mx.quantize_grouped(use, rw, True, columnwise_transposed=True)
        for x, p in zip(use, got):
            single = mx.quantize(x, rw, True, columnwise_transposed=True)
            torch.cuda.synchronize()
            for a, b in zip(p, single):
                if a is not None:
                    assert torch.equal(a, b)


def test_input_gradient_from_f32_master_weight(orc):
    """dx = dy . w with w's transposed columnwise plane quantized from its
    float32 master copy, against the float64 product of the untransposed
    planes."""
    T, N, K = 256, 512, 768
    g = torch.Generator().manual_seed(55)
    w = torch.randn(N, K, generator=g) * 0.05
    dy = (torch.randn(T, N, generator=g) * 0.01).to(torch.bfloat16)
    say("input gradient from a float32 master weight", (T, N, K))
    pw = mx.quantize(w.to(DEV), False, True, columnwise_transposed=True)
    pdy = mx.quantize(dy.to(DEV), True, False)
    dx = mx.gemm(pdy.rowwise_data, pdy.rowwise_scale, pw.columnwise_data, pw.columnwise_scale, torch.float32)
    torch.cuda.synchronize()
    qc, sc = orc.quantize_colwise(w.numpy())
    q, s = orc.quantize_rowwise(synth.bf16_bits(dy))
    ref = orc.dequantize(q, s, 0) @ orc.dequantize(qc, sc, 1)
    hp = [host(t) for t in (pdy.rowwise_data, pdy.rowwise_scale, pw.columnwise_data, pw.columnwise_scale)]
    C, mag = orc.gemm(*hp)
    assert (np.abs(C - ref) <= 1e-12 * mag).all(), "the planes do not hold w^T"
    err = np.abs(host(dx).astype(np.float64) - C)
    assert (err <= acc.bound(*hp)).all()


# the products take the skinny row blocks and, for the input gradient of
# (1024, 512, 1024), the ring tiles
@pytest.mark.parametrize("tnk", [(256, 384, 512), (512, 768, 640), (1024, 512, 1024)])
def test_backward_products(orc, tnk):
    """A linear layer y = x w^T with x [T, K], w [N, K] and the gradient dy
    [T, N], all quantized once with both planes (columnwise transposed):
      input gradient  dx [T, K] = dy . w: A = dy rowwise, B = w's columnwise plane;
      weight gradient dw [N, K] = dy^T . x: A = dy's columnwise plane, B = x's.
    Each product is within the accumulation bound of the oracle's float64
    product of the same planes, and that float64 product equals the one
    computed from the untransposed columnwise planes of the same tensors,
    dequantized by the oracle (so the transposed planes mean w^T, dy^T and
    x^T)."""
    T, N, K = tnk
    g = torch.Generator().manual_seed(T + N + K)
    x = torch.randn(T, K, generator=g).to(torch.bfloat16)
    w = (torch.randn(N, K, generator=g) * 0.05).to(torch.bfloat16)
    dy = (torch.randn(T, N, generator=g) * 0.01).to(torch.bfloat16)
    say("backward products", tnk)
    px, pw, pdy = (mx.quantize(t.to(DEV), True, True, columnwise_transposed=True) for t in (x, w, dy))
    dx = mx.gemm(pdy.rowwise_data, pdy.rowwise_scale, pw.columnwise_data, pw.columnwise_scale, torch.float32)
    dw = mx.gemm(pdy.columnwise_data, pdy.columnwise_scale, px.columnwise_data, px.columnwise_scale,
                 torch.float32)
    torch.cuda.synchronize()
    assert tuple(dx.shape) == (T, K) and tuple(dw.shape) == (N, K)

    def deq_col(t):
        q, s = orc.quantize_colwise(synth.bf16_bits(t))
        return orc.dequantize(q, s, 1)            # float64 [rows, cols]

    def deq_row(t):
        q, s = orc.quantize_rowwise(synth.bf16_bits(t))
        return orc.dequantize(q, s, 0)

    for got, planes, ref, what in (
            (dx, (pdy.rowwise_data, pdy.rowwise_scale, pw.columnwise_data, pw.columnwise_scale),
             deq_row(dy) @ deq_col(w), "input gradient"),
            (dw, (pdy.columnwise_data, pdy.columnwise_scale, px.columnwise_data, px.columnwise_scale),
             deq_col(dy).T @ deq_col(x), "weight gradient")):
        hp = [host(t) for t in planes]
        C, mag = orc.gemm(*hp)
        # both float64 sums of the same exact products, in different orders
        assert (np.abs(C - ref) <= 1e-12 * mag).all(), "%s: the planes do not hold the transposes" % what
        tol = acc.bound(*hp)
        err = np.abs(host(got).astype(np.float64) - C)
        assert (err <= tol).all(), "%s: %d outputs beyond the bound" % (what, int((err > tol).sum()))

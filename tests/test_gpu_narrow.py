"""Columnwise planes of tensors whose rows are not a multiple of 8 elements
(the narrow path: one thread per column of a 32-row block, element-sized
accesses), for bf16 and float32 input and for dequantize, against the oracle
byte for byte; inside guard bands, with padded scale rows, and mixed with
tiled tensors in one grouped launch."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_02_amd as mx
from tests import oracle_pins as P
from tests.test_gpu_parity import (DEV, assert_guards, assert_same, dev_bits, dev_f32, f32_specials,
                                   guarded, host, say, special_values)

pytestmark = pytest.mark.gpu

NARROW = [(32, 1), (32, 7), (64, 13), (96, 1001), (32, 263), (160, 517), (4096, 4095)]


@pytest.mark.parametrize("shape", NARROW)
def test_bf16_columnwise(orc, shape):
    rows, cols = shape
    bits = special_values(rows, cols, seed=rows * 7 + cols)
    say("narrow bf16", shape)
    p = mx.quantize(dev_bits(bits), rowwise=False, columnwise=True)
    torch.cuda.synchronize()
    qc, sc = orc.quantize_colwise(bits)
    assert_same(host(p.columnwise_data), qc, "narrow q_col %s" % (shape,))
    assert_same(host(p.columnwise_scale), sc, "narrow s_col %s" % (shape,))


def test_bf16_columnwise_random_tensors(orc):
    for i, b in enumerate(P.random_tensors(seed=5, rows=64, cols=75)):
        say("narrow bf16 random", i)
        p = mx.quantize(dev_bits(b), rowwise=False, columnwise=True)
        torch.cuda.synchronize()
        qc, sc = orc.quantize_colwise(b)
        assert_same(host(p.columnwise_data), qc, "narrow random %d q_col" % i)
        assert_same(host(p.columnwise_scale), sc, "narrow random %d s_col" % i)


@pytest.mark.parametrize("shape", [(32, 5), (64, 1001), (96, 263)])
def test_f32_columnwise(orc, shape):
    x = f32_specials(*shape, seed=shape[1])
    say("narrow f32", shape)
    p = mx.quantize(dev_f32(x), rowwise=False, columnwise=True)
    torch.cuda.synchronize()
    qc, sc = orc.quantize_colwise(x)
    assert_same(host(p.columnwise_data), qc, "narrow f32 q_col %s" % (shape,))
    assert_same(host(p.columnwise_scale), sc, "narrow f32 s_col %s" % (shape,))


def test_grouped_mixes_narrow_and_tiled(orc):
    """One grouped launch through the C ABI with per-tensor requests: narrow
    columnwise, tiled row + column, tiled columnwise-only and more narrow
    tensors."""
    shapes = [(64, 1001), (64, 1024), (32, 37), (96, 512), (32, 3)]
    reqs = [(False, True), (True, True), (False, True), (False, True), (False, True)]
    bits = [special_values(r, c, seed=r + c) for r, c in shapes]
    xs = [dev_bits(b) for b in bits]
    descs, planes = [], []
    for x, (row, col) in zip(xs, reqs):
        d, pl = mx._quant_desc(x, row, col, None)
        descs.append(d)
        planes.append(pl)
    say("narrow grouped mixed")
    arr = (mx._QuantDesc * len(descs))(*descs)
    mx._check(mx.lib().mxfp8_quantize_grouped(arr, len(descs), torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    for b, pl, (row, col), shape in zip(bits, planes, reqs, shapes):
        qc, sc = orc.quantize_colwise(b)
        assert_same(host(pl.columnwise_data), qc, "mixed q_col %s" % (shape,))
        assert_same(host(pl.columnwise_scale), sc, "mixed s_col %s" % (shape,))
        if row:
            qr, sr = orc.quantize_rowwise(b)
            assert_same(host(pl.rowwise_data), qr, "mixed q_row %s" % (shape,))
            assert_same(host(pl.rowwise_scale), sr, "mixed s_row %s" % (shape,))


@pytest.mark.parametrize("shape", [(32, 7), (96, 1001)])
def test_guard_bands_and_odd_scale_pitch(orc, shape):
    """q_col inside 0xA5 guard bands, s_col rows 3 bytes apart beyond the
    plane's width (an odd pitch)."""
    rows, cols = shape
    bits = special_values(rows, cols, seed=cols)
    qbuf, q = guarded(rows * cols, torch.uint8)
    srows = rows // 32
    sbuf = torch.full((4096 + srows * (cols + 3) + 4096,), 0xA5, dtype=torch.uint8, device=DEV)
    s = sbuf[4096:4096 + srows * (cols + 3)].view(srows, cols + 3)[:, :cols]
    say("narrow guarded", shape)
    mx.quantize(dev_bits(bits), False, True, out=mx.MXFP8Planes(None, q.view(rows, cols), None, s))
    torch.cuda.synchronize()
    assert_guards(qbuf, what="narrow q_col")
    sb = host(sbuf)
    inside = np.zeros(sb.size, bool)
    inside[4096:4096 + srows * (cols + 3)].reshape(srows, cols + 3)[:, :cols] = True
    assert (sb[~inside] == 0xA5).all(), "narrow s_col: write outside the plane"
    qc, sc = orc.quantize_colwise(bits)
    assert_same(host(q.view(rows, cols)), qc, "guarded q_col")
    assert_same(host(s), sc, "guarded s_col")


@pytest.mark.parametrize("shape", [(32, 7), (96, 1001), (64, 263)])
def test_dequantize_columnwise(orc, shape):
    rows, cols = shape
    bits = special_values(rows, cols, seed=cols + 1)
    p = mx.quantize(dev_bits(bits), False, True)
    ref = orc.dequantize(host(p.columnwise_data), host(p.columnwise_scale), mx.COLUMNWISE)
    for dtype in (torch.float32, torch.bfloat16):
        say("narrow dequantize", shape, dtype)
        buf, out = guarded(rows * cols, dtype)
        mx.dequantize(p.columnwise_data, p.columnwise_scale, mx.COLUMNWISE, dtype, out=out.view(rows, cols))
        torch.cuda.synchronize()
        assert_guards(buf, what="narrow dequantize %s" % dtype)
        got = host(out.view(rows, cols).float()).astype(np.float64)
        want = ref if dtype == torch.float32 else P.bf16_values(orc.round_bf16(ref))
        assert ((got == want) | (np.isnan(got) & np.isnan(want))).all()
    # every code under every scale byte, 3 columns wide
    q = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(256, 1).repeat(1, 3).contiguous().to(DEV)
    s = torch.arange(8, dtype=torch.int32).to(torch.uint8).view(8, 1).repeat(1, 3).contiguous().to(DEV) * 31
    got = host(mx.dequantize(q, s, mx.COLUMNWISE, torch.float32)).astype(np.float64)
    want = orc.dequantize(host(q), host(s), mx.COLUMNWISE)
    assert ((got == want) | (np.isnan(got) & np.isnan(want))).all()

"""Tensors of more than 2^31 elements: every kernel's addressing past 2 GiB of
fp8 plane and 4 GiB of bf16 input.  Each launch covers the whole tensor; 32-row
strips at the start, the middle and the end (and sampled outputs of the matrix
products) are checked against the oracle."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_02_amd as mx
from mxfp8_block_scaled_02_amd import synth
from tests import gemm_accuracy as acc
from tests import oracle_pins as P
from tests.test_gpu_parity import DEV, assert_same, check_fused_out, host, say

pytestmark = pytest.mark.gpu

# 2^31 + 2^21 elements: the last strips start past element 2^31
ROWS, COLS = 65536 + 64, 32768


def strips(rows):
    """First rows of 32-row strips: the start, the middle, the end."""
    return (0, (rows // 64) * 32, rows - 32)


def big(rows, cols, seed, dtype=torch.bfloat16, std=1.0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    x = torch.empty((rows, cols), dtype=dtype, device=DEV)
    x.normal_(0.0, std, generator=g)
    return x


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def check_planes(orc, x_strip, p, r0, row, col, what):
    if row:
        qr, sr = orc.quantize_rowwise(x_strip)
        assert_same(host(p.rowwise_data[r0:r0 + 32]), qr, "%s q_row rows %d.." % (what, r0))
        assert_same(host(p.rowwise_scale[r0:r0 + 32]), sr, "%s s_row rows %d.." % (what, r0))
    if col:
        qc, sc = orc.quantize_colwise(x_strip)
        assert_same(host(p.columnwise_data[r0:r0 + 32]), qc, "%s q_col rows %d.." % (what, r0))
        assert_same(host(p.columnwise_scale[r0 // 32:r0 // 32 + 1]), sc, "%s s_col block %d" % (what, r0 // 32))


def test_quantize_bf16(orc):
    """Row + column tiles, column tiles alone and the flat rowwise path."""
    x = big(ROWS, COLS, 1)
    for row, col in ((True, True), (False, True), (True, False)):
        say("large quantize bf16", (ROWS, COLS), row, col)
        p = mx.quantize(x, row, col)
        torch.cuda.synchronize()
        for r0 in strips(ROWS):
            check_planes(orc, synth.bf16_bits(x[r0:r0 + 32]), p, r0, row, col, "bf16")
        del p


def test_quantize_bf16_transposed_columnwise(orc):
    """The columnwise plane stored transposed, [32768, 65600]: its rows'
    offsets pass 2^31 (and the rowwise plane of the same launch)."""
    x = big(ROWS, COLS, 1)
    say("large quantize bf16, transposed columnwise", (ROWS, COLS))
    p = mx.quantize(x, True, True, columnwise_transposed=True)
    torch.cuda.synchronize()
    for r0 in strips(ROWS):
        bits = synth.bf16_bits(x[r0:r0 + 32])
        check_planes(orc, bits, p, r0, True, False, "bf16 transposed")
        qc, sc = orc.quantize_colwise(bits)
        assert_same(host(p.columnwise_data[:, r0:r0 + 32]), np.ascontiguousarray(qc.T),
                    "q_colT rows %d.." % r0)
        assert_same(host(p.columnwise_scale[:, r0 // 32]), sc[0], "s_colT block %d" % (r0 // 32))


def test_quantize_f32_transposed_columnwise(orc):
    """float32 input [65600, 32768] (8.6 GB), the columnwise plane stored
    transposed: its rows' offsets pass 2^31."""
    x = big(ROWS, COLS, 11, torch.float32, 0.02)
    say("large quantize f32, transposed columnwise", (ROWS, COLS))
    p = mx.quantize(x, False, True, columnwise_transposed=True)
    torch.cuda.synchronize()
    for r0 in strips(ROWS):
        qc, sc = orc.quantize_colwise(host(x[r0:r0 + 32]))
        assert_same(host(p.columnwise_data[:, r0:r0 + 32]), np.ascontiguousarray(qc.T),
                    "f32 q_colT rows %d.." % r0)
        assert_same(host(p.columnwise_scale[:, r0 // 32]), sc[0], "f32 s_colT block %d" % (r0 // 32))


def test_quantize_f32(orc):
    x = big(ROWS, COLS, 2, torch.float32, 0.02)
    for row, col in ((True, True), (True, False)):
        say("large quantize f32", (ROWS, COLS), row, col)
        p = mx.quantize(x, row, col)
        torch.cuda.synchronize()
        for r0 in strips(ROWS):
            check_planes(orc, host(x[r0:r0 + 32]), p, r0, row, col, "f32")
        del p


@pytest.mark.parametrize("shape", [(262144 + 64, 8192), (ROWS, COLS)])
def test_rmsnorm_quantize(orc, shape):
    """Rows held in registers (8192 columns, two rows per task) and rows read
    twice (32768 columns)."""
    rows, cols = shape
    x = big(rows, cols, 3, std=3.0)
    gamma = big(1, cols, 4).reshape(cols).mul_(0.1).add_(1.0)
    say("large rmsnorm", shape)
    normed, q, s = mx.rmsnorm_quantize(x, gamma, 1.0, 1e-6)
    torch.cuda.synchronize()
    gb = synth.bf16_bits(gamma)
    for r0 in (0, rows // 2, rows - 4):          # four rows each; the last ends the tensor
        sl = slice(r0, r0 + 4)
        check_fused_out(orc, synth.bf16_bits(x[sl]), gb, 1.0, 1e-6, synth.bf16_bits(normed[sl]),
                        host(q[sl]), host(s[sl]), "large rmsnorm %s rows %d.." % (shape, sl.start))


def test_dequantize(orc):
    x = big(ROWS, COLS, 5)
    p = mx.quantize(x, True, True)
    del x
    for axis, q, s, dtype in ((mx.ROWWISE, p.rowwise_data, p.rowwise_scale, torch.float32),
                              (mx.COLUMNWISE, p.columnwise_data, p.columnwise_scale, torch.bfloat16)):
        say("large dequantize", (ROWS, COLS), axis, dtype)
        out = mx.dequantize(q, s, axis, dtype)
        torch.cuda.synchronize()
        for r0 in strips(ROWS):
            qs = host(q[r0:r0 + 32])
            ss = host(s[r0:r0 + 32] if axis == mx.ROWWISE else s[r0 // 32:r0 // 32 + 1])
            want = orc.dequantize(qs, ss, axis)
            if dtype == torch.bfloat16:
                want = P.bf16_values(orc.round_bf16(want))
            got = host(out[r0:r0 + 32].float()).astype(np.float64)
            assert ((got == want) | (np.isnan(got) & np.isnan(want))).all(), "dequantize rows %d.." % r0
        del out


def random_planes(rows, K, seed):
    """Random fp8 codes (no NaN) and scale bytes around 2^0, on the device."""
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randint(0, 256, (rows, K), dtype=torch.uint8, device=DEV, generator=g)
    q[(q & 0x7F) == 0x7F] = 0x38
    s = torch.randint(120, 134, (rows, K // 32), dtype=torch.uint8, device=DEV, generator=g)
    return q, s


def check_products(orc, qa, sa, qb, sb, out, ms, ns, what):
    planes = [host(t) for t in (qa[ms], sa[ms], qb[ns], sb[ns])]
    C, _ = orc.gemm(*planes)
    mm, nn = np.meshgrid(np.arange(len(ms)), np.arange(len(ns)), indexing="ij")
    tol = acc.bound_at(*planes, mm.ravel(), nn.ravel()).reshape(C.shape)
    got = host(out[ms][:, ns]).astype(np.float64)
    bad = np.abs(got - C) > tol
    assert not bad.any(), "%s: %d of %d outputs outside the bound" % (what, int(bad.sum()), bad.size)


def test_gemm_ring_tiles(orc):
    """A [65600, 32768]: the ring tiles' A offsets pass 2^31."""
    M, N, K = ROWS, 256, COLS
    qa, sa = random_planes(M, K, 6)
    qb, sb = random_planes(N, K, 7)
    say("large gemm ring", (M, N, K))
    out = mx.gemm(qa, sa, qb, sb, torch.float32)
    torch.cuda.synchronize()
    ms = torch.tensor([0, 1, M // 2, M - 33, M - 2, M - 1], device=DEV)
    ns = torch.tensor([0, 37, 128, 255], device=DEV)
    check_products(orc, qa, sa, qb, sb, out, ms, ns, "ring")


def test_gemm_grouped_ring_tiles(orc):
    """The same A [65600, 32768] as one product of a grouped call (its ring
    tiles in a launch table), and a 16-row product beside it."""
    M, N, K = ROWS, 256, COLS
    qa, sa = random_planes(M, K, 6)
    qb, sb = random_planes(N, K, 7)
    qc, sc = random_planes(16, K, 10)
    say("large gemm grouped", (M, N, K), (16, N, K))
    out, small = mx.gemm_grouped([qa, qc], [sa, sc], [qb, qb], [sb, sb], torch.float32)
    torch.cuda.synchronize()
    ms = torch.tensor([0, 1, M // 2, M - 33, M - 2, M - 1], device=DEV)
    ns = torch.tensor([0, 37, 128, 255], device=DEV)
    check_products(orc, qa, sa, qb, sb, out, ms, ns, "grouped ring")
    check_products(orc, qc, sc, qb, sb, small, torch.tensor([0, 15], device=DEV), ns, "grouped skinny")


def test_gemm_skinny(orc):
    """B [65600, 32768] under 16 activation rows: the skinny kernel's B
    offsets pass 2^31."""
    M, N, K = 16, ROWS, COLS
    qa, sa = random_planes(M, K, 8)
    qb, sb = random_planes(N, K, 9)
    say("large gemm skinny", (M, N, K))
    out = mx.gemm(qa, sa, qb, sb, torch.float32)
    torch.cuda.synchronize()
    ms = torch.tensor([0, 7, 15], device=DEV)
    ns = torch.tensor([0, 1, N // 2, N - 33, N - 2, N - 1], device=DEV)
    check_products(orc, qa, sa, qb, sb, out, ms, ns, "skinny")

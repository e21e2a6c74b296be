"""GPU parity: the HIP library, called through its C ABI, against the CPU
oracle on the same seeded inputs.

Quantized bytes and scales must match bit for bit; dequantized values must be
equal (NaN where NaN); the fused op's normed bf16 must be within 2^-7 of the
oracle's float64 RMSNorm (relative, zero exactly where the oracle's is zero),
and its bytes must equal the oracle's quantize of the GPU's own normed output.
"""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_02_amd as mx
from mxfp8_block_scaled_02_amd import synth
from tests import oracle_pins as P

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print("[case]", *a, flush=True)


def dev_bits(bits: np.ndarray) -> torch.Tensor:
    """bf16 GPU tensor with the given uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy())
    return t.view(torch.bfloat16).to(DEV)


def host(t):
    return None if t is None else t.cpu().numpy()


def assert_same(got, want, what):
    assert got.shape == want.shape, "%s: shape %s vs %s" % (what, got.shape, want.shape)
    bad = got != want
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d of %d bytes differ, first at %s: got %s want %s" % (
            what, int(bad.sum()), bad.size, idx.tolist(),
            [hex(int(got[tuple(i)])) for i in idx], [hex(int(want[tuple(i)])) for i in idx]))


def check_quantize(orc, bits, rowwise=True, columnwise=True, what=""):
    say("quantize", what, bits.shape, "row" if rowwise else "", "col" if columnwise else "")
    planes = mx.quantize(dev_bits(bits), rowwise=rowwise, columnwise=columnwise)
    torch.cuda.synchronize()
    if rowwise:
        qr, sr = orc.quantize_rowwise(bits)
        assert_same(host(planes.rowwise_data), qr, what + " q_row")
        assert_same(host(planes.rowwise_scale), sr, what + " s_row")
    if columnwise:
        qc, sc = orc.quantize_colwise(bits)
        assert_same(host(planes.columnwise_data), qc, what + " q_col")
        assert_same(host(planes.columnwise_scale), sc, what + " s_col")
    return planes


def special_values(rows, cols, seed):
    """Random bits with NaN/Inf blocks, zeros, subnormals and saturating values."""
    g = np.random.default_rng(seed)
    x = P.bf16_bits_of(np.zeros(1))[0] + np.zeros((rows, cols), np.uint16)
    normal = torch.randn(rows, cols, generator=torch.Generator().manual_seed(seed))
    x[:] = normal.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for _ in range(max(1, rows * cols // 512)):
        r, c = g.integers(rows), g.integers(cols)
        x[r, c] = g.choice([0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x0001, 0x8001, 0x0000, 0x8000,
                            0x7F7F, 0xFF7F, 0x43E8, 0xC3F0])   # 464, -480
    return x


# ---------------------------------------------------------------- quantize --

SMALL_SHAPES = [(32, 32), (32, 64), (64, 544), (96, 1056), (32, 4128), (160, 96), (256, 1024)]


@pytest.mark.parametrize("shape", SMALL_SHAPES)
def test_row_and_col_small(orc, shape):
    for i, bits in enumerate(P.random_tensors(seed=shape[0] + shape[1], rows=shape[0], cols=shape[1])):
        check_quantize(orc, bits, True, True, "random%d" % i)
    check_quantize(orc, special_values(*shape, seed=3), True, True, "specials")


@pytest.mark.parametrize("shape", [(1, 32), (3, 96), (7, 4128), (33, 544), (1000, 64)])
def test_rowwise_only_ragged(orc, shape):
    # flat path with partial last tasks; rows need not be a multiple of 32
    for i, bits in enumerate(P.random_tensors(seed=7, rows=shape[0], cols=shape[1])):
        check_quantize(orc, bits, True, False, "rowonly%d" % i)


@pytest.mark.parametrize("shape", [(4095, 2048), (4096, 2048), (4097, 2080)])
def test_rowwise_only_around_the_unroll_switch(orc, shape):
    # just below 2^20 8-element pieces a lane takes one piece per task, from
    # there on four (the last of these shapes also ends in a partial task)
    for i, bits in enumerate(P.random_tensors(seed=11, rows=shape[0], cols=shape[1])[:2]):
        check_quantize(orc, bits, True, False, "rowonly-switch%d" % i)


@pytest.mark.parametrize("shape", [(32, 8), (64, 40), (32, 520), (96, 1000)])
def test_columnwise_only_cols_multiple_of_8(orc, shape):
    for i, bits in enumerate(P.random_tensors(seed=9, rows=shape[0], cols=shape[1])):
        check_quantize(orc, bits, False, True, "colonly%d" % i)


def test_rowwise_workload_256x1024(orc):
    x = synth.workload("rowwise_256x1024")["x"]
    check_quantize(orc, synth.bf16_bits(x), True, False, "rowwise_256x1024")


def test_every_bf16_value_as_a_block(orc):
    pats = P.all_bf16_patterns()
    n = pats.size
    x = np.zeros((n, 32), np.uint16)
    x[np.arange(n), np.arange(n) % 32] = pats
    check_quantize(orc, x, True, False, "single-value rows")
    check_quantize(orc, np.ascontiguousarray(x[:, :].T[:, : 65536 // 2]), True, True,
                   "single-value columns (first half)")
    check_quantize(orc, np.ascontiguousarray(x.T[:, 65536 // 2:]), True, True,
                   "single-value columns (second half)")


def test_every_value_against_every_scale(orc):
    x, _ = P.pair_blocks()
    rows = x.shape[0] - x.shape[0] % 32
    check_quantize(orc, x[:rows], True, False, "pairs rowwise")
    xt = np.ascontiguousarray(x[:rows].T)          # the same blocks down columns
    cols = xt.shape[1] - xt.shape[1] % 8
    check_quantize(orc, np.ascontiguousarray(xt[:, :cols]), False, True, "pairs columnwise")


def test_rowwise_activation_8192x7168_full(orc):
    # the rowwise-only bench workload at full size, every byte against the oracle
    x = synth.workload("rowwise_8192x7168")["x"]
    check_quantize(orc, synth.bf16_bits(x), True, False, "activation 8192x7168")


def test_weight_4096_full(orc):
    x = synth.workload("rowcol_4096x4096")["x"]
    check_quantize(orc, synth.bf16_bits(x), True, True, "rowcol_4096x4096")


def test_determinism_and_in_place_outputs(orc):
    x = dev_bits(special_values(256, 2048, seed=4))
    a = mx.quantize(x, True, True)
    ptrs = [t.data_ptr() for t in a]
    first = [host(t).copy() for t in a]
    b = mx.quantize(x, True, True, out=a)           # persistent buffers, rewritten in place
    torch.cuda.synchronize()
    assert [t.data_ptr() for t in b] == ptrs
    for f, t in zip(first, b):
        assert np.array_equal(f, host(t))


def test_guard_bands(orc):
    rows, cols = 96, 1056
    bits = special_values(rows, cols, seed=12)
    pad = 4096
    bufs = [torch.full((rows * cols + 2 * pad,), 0xA5, dtype=torch.uint8, device=DEV) for _ in range(2)]
    sbufs = [torch.full((rows * cols // 32 + 2 * pad,), 0x5A, dtype=torch.uint8, device=DEV) for _ in range(2)]
    out = mx.MXFP8Planes(bufs[0][pad:pad + rows * cols].view(rows, cols),
                         bufs[1][pad:pad + rows * cols].view(rows, cols),
                         sbufs[0][pad:pad + rows * cols // 32].view(rows, cols // 32),
                         sbufs[1][pad:pad + rows * cols // 32].view(rows // 32, cols))
    mx.quantize(dev_bits(bits), True, True, out=out)
    torch.cuda.synchronize()
    for b, fill in ((bufs[0], 0xA5), (bufs[1], 0xA5), (sbufs[0], 0x5A), (sbufs[1], 0x5A)):
        h = host(b)
        assert (h[:pad] == fill).all() and (h[-pad:] == fill).all(), "write outside the plane"
    qr, sr = orc.quantize_rowwise(bits)
    assert_same(host(out.rowwise_data), qr, "guarded q_row")


def test_empty_tensor_is_a_no_op():
    x = torch.empty((0, 1024), dtype=torch.bfloat16, device=DEV)
    p = mx.quantize(x, True, True)
    assert p.rowwise_data.shape == (0, 1024)


# ------------------------------------------------ float32 master weights --

def f32_specials(rows, cols, seed):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((rows, cols)) * np.ldexp(1.0, g.integers(-30, 30, (rows, 1)))).astype(np.float32)
    bits = x.view(np.uint32)
    for _ in range(max(1, rows * cols // 512)):
        r, c = g.integers(rows), g.integers(cols)
        bits[r, c] = g.choice([0x7F800000, 0xFF800000, 0x7FC00000, 0xFFC00001, 0x00000001, 0x80000001,
                               0x00000000, 0x80000000, 0x7F7FFFFF, 0xFF7FFFFF, 0x00400000, 0x007FFFFF])
    return x


def dev_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def check_quantize_f32(orc, x, rowwise=True, columnwise=True, what=""):
    say("quantize_f32", what, x.shape, "row" if rowwise else "", "col" if columnwise else "")
    planes = mx.quantize(dev_f32(x), rowwise=rowwise, columnwise=columnwise)
    torch.cuda.synchronize()
    if rowwise:
        qr, sr = orc.quantize_rowwise(x)
        assert_same(host(planes.rowwise_data), qr, what + " q_row")
        assert_same(host(planes.rowwise_scale), sr, what + " s_row")
    if columnwise:
        qc, sc = orc.quantize_colwise(x)
        assert_same(host(planes.columnwise_data), qc, what + " q_col")
        assert_same(host(planes.columnwise_scale), sc, what + " s_col")


@pytest.mark.parametrize("shape", [(32, 32), (64, 544), (96, 1056), (32, 4128), (160, 96)])
def test_f32_row_and_col(orc, shape):
    check_quantize_f32(orc, f32_specials(*shape, seed=shape[1]), True, True, "f32 specials")
    for i, b in enumerate(P.random_tensors(seed=3, rows=shape[0], cols=shape[1])):
        check_quantize_f32(orc, P.bf16_values(b).astype(np.float32), True, True, "f32 from bf16 %d" % i)


def test_f32_ties_and_wide_range(orc):
    x = P.f32_blocks()
    rows = x.shape[0] - x.shape[0] % 32
    check_quantize_f32(orc, x[:rows], True, False, "f32 blocks rowwise")
    check_quantize_f32(orc, np.ascontiguousarray(x[:rows].T), False, True, "f32 blocks columnwise")


@pytest.mark.parametrize("shape", [(1, 32), (3, 96), (7, 4128), (1000, 64)])
def test_f32_rowwise_only_ragged(orc, shape):
    check_quantize_f32(orc, f32_specials(*shape, seed=11), True, False, "f32 rowonly")


@pytest.mark.parametrize("shape", [(32, 8), (64, 40), (96, 1000)])
def test_f32_columnwise_only(orc, shape):
    check_quantize_f32(orc, f32_specials(*shape, seed=12), False, True, "f32 colonly")


def test_f32_master_weight_4096(orc):
    x = synth.workload("rowcol_f32_4096x4096", device=DEV)["x"]
    check_quantize_f32(orc, x.cpu().numpy(), True, True, "rowcol_f32_4096x4096")


def test_f32_grouped_equals_single(orc):
    shapes = [(32, 256), (64, 544), (96, 7168), (32, 40)]
    xs = [f32_specials(*sh, seed=60 + i) for i, sh in enumerate(shapes)]
    planes = mx.quantize_grouped([dev_f32(x) for x in xs], False, True)
    torch.cuda.synchronize()
    for x, p in zip(xs, planes):
        qc, sc = orc.quantize_colwise(x)
        assert_same(host(p.columnwise_data), qc, "grouped f32 q_col")
        assert_same(host(p.columnwise_scale), sc, "grouped f32 s_col")


# ------------------------------------------------------------------ grouped --

def test_grouped_mixed_shapes_equal_single_calls(orc):
    shapes = [(32, 32), (64, 544), (96, 7168), (32, 4128), (128, 96), (32, 8 * 65)]
    g = torch.Generator().manual_seed(21)
    xs = [(torch.randn(s, generator=g) * 10 ** (i - 3)).to(torch.bfloat16) for i, s in enumerate(shapes)]
    say("grouped", shapes)
    for rowwise, columnwise in ((True, True), (True, False), (False, True)):
        use = [x for x in xs if (not rowwise or x.shape[1] % 32 == 0)]
        planes = mx.quantize_grouped([x.to(DEV) for x in use], rowwise, columnwise)
        torch.cuda.synchronize()
        for x, p in zip(use, planes):
            bits = synth.bf16_bits(x)
            single = mx.quantize(x.to(DEV), rowwise, columnwise)
            torch.cuda.synchronize()
            for a, b in zip(p, single):
                if a is not None:
                    assert np.array_equal(host(a), host(b))
            if rowwise:
                qr, sr = orc.quantize_rowwise(bits)
                assert_same(host(p.rowwise_data), qr, "grouped q_row")
                assert_same(host(p.rowwise_scale), sr, "grouped s_row")
            if columnwise:
                qc, sc = orc.quantize_colwise(bits)
                assert_same(host(p.columnwise_data), qc, "grouped q_col")
                assert_same(host(p.columnwise_scale), sc, "grouped s_col")


def test_grouped_more_than_one_launch(orc):
    # 70 tensors: more than one argument block per call
    g = torch.Generator().manual_seed(5)
    xs = [torch.randn((32, 32 * (1 + i % 5)), generator=g).to(torch.bfloat16) for i in range(70)]
    say("grouped 70 tensors")
    planes = mx.quantize_grouped([x.to(DEV) for x in xs], True, True)
    torch.cuda.synchronize()
    for x, p in zip(xs, planes):
        bits = synth.bf16_bits(x)
        qr, sr = orc.quantize_rowwise(bits)
        qc, sc = orc.quantize_colwise(bits)
        assert_same(host(p.rowwise_data), qr, "q_row")
        assert_same(host(p.columnwise_scale), sc, "s_col")
        assert_same(host(p.columnwise_data), qc, "q_col")
        assert_same(host(p.rowwise_scale), sr, "s_row")


def test_grouped_64_experts_full_size(orc):
    say("grouped_64x2048x7168 on device")
    xs = synth.workload("grouped_64x2048x7168", device=DEV)["xs"]
    planes = mx.quantize_grouped(xs, True, True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    full = {0, 63, int(rng.integers(1, 63))}
    for i, (x, p) in enumerate(zip(xs, planes)):
        if i in full:
            bits = synth.bf16_bits(x)
            say("expert", i, "full compare")
        else:
            # one random 32-row block strip, all columns, of every other expert
            r0 = 32 * int(rng.integers(0, x.shape[0] // 32))
            bits = synth.bf16_bits(x[r0:r0 + 32])
            p = mx.MXFP8Planes(p.rowwise_data[r0:r0 + 32], p.columnwise_data[r0:r0 + 32],
                               p.rowwise_scale[r0:r0 + 32], p.columnwise_scale[r0 // 32:r0 // 32 + 1])
        qr, sr = orc.quantize_rowwise(bits)
        qc, sc = orc.quantize_colwise(bits)
        assert_same(host(p.rowwise_data), qr, "expert %d q_row" % i)
        assert_same(host(p.rowwise_scale), sr, "expert %d s_row" % i)
        assert_same(host(p.columnwise_data), qc, "expert %d q_col" % i)
        assert_same(host(p.columnwise_scale), sc, "expert %d s_col" % i)


# ----------------------------------------------------------------- RMSNorm --

def check_fused(orc, x, gamma, off, eps, rows_sel=None, what=""):
    say("rmsnorm_quantize", what, tuple(x.shape))
    normed, q, s = mx.rmsnorm_quantize(x, gamma, off, eps)
    torch.cuda.synchronize()
    xb = synth.bf16_bits(x if rows_sel is None else x[rows_sel])
    gb = synth.bf16_bits(gamma)
    nb = synth.bf16_bits(normed if rows_sel is None else normed[rows_sel])
    qg = host(q if rows_sel is None else q[rows_sel])
    sg = host(s if rows_sel is None else s[rows_sel])
    ref = orc.rmsnorm_f64(xb, gb, off, eps)
    got = P.bf16_values(nb)
    assert ((got == 0) == (ref == 0)).all(), what + ": zero pattern"
    rel_ok = np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref)
    assert rel_ok.all(), "%s: normed off by more than 2^-7 at %d places" % (what, int((~rel_ok).sum()))
    q2, s2 = orc.quantize_rowwise(nb)            # byte identity with a standalone quantize
    assert_same(qg, q2, what + " q")
    assert_same(sg, s2, what + " s")
    return normed, q, s


@pytest.mark.parametrize("shape", [(1, 32), (5, 96), (16, 512), (3, 544), (64, 4096),
                                   (8, 16384), (4, 16416), (2, 40000),
                                   # at most 256 rows: 16 waves per row (1 or 2 chunks a
                                   # lane); 257 rows: four waves per row again
                                   (3, 12288), (256, 2080), (257, 2080),
                                   # enough rows that a workgroup walks several, last group ragged
                                   (2051, 96), (4099, 2048), (16411, 4096), (20003, 7168)])
def test_fused_shapes(orc, shape):
    x, gamma = synth.rmsnorm_inputs(*shape, seed=shape[1], x_std=2.0, row_decades=1.5)
    check_fused(orc, x.to(DEV), gamma.to(DEV), 0.5, 1e-5, what="shape %s" % (shape,))


def test_fused_equals_standalone_quantize_on_gpu(orc):
    x, gamma = synth.rmsnorm_inputs(64, 7168, seed=2, x_std=3.0, row_decades=2.0)
    normed, q, s = mx.rmsnorm_quantize(x.to(DEV), gamma.to(DEV), 0.0, 1e-5)
    p = mx.quantize(normed, True, False)
    torch.cuda.synchronize()
    assert np.array_equal(host(q), host(p.rowwise_data))
    assert np.array_equal(host(s), host(p.rowwise_scale))
    n2, q2, s2 = mx.rmsnorm_quantize(x.to(DEV), gamma.to(DEV), 0.0, 1e-5)
    torch.cuda.synchronize()
    assert np.array_equal(host(n2.view(torch.int16)), host(normed.view(torch.int16)))


def test_fused_workload_8192(orc):
    w = synth.workload("rmsnorm_8192x8192", device=DEV)
    check_fused(orc, w["x"], w["gamma"], w["weight_offset"], w["eps"], what="rmsnorm_8192x8192")


def test_fused_workload_decode(orc):
    w = synth.workload("rmsnorm_decode_16x7168")
    check_fused(orc, w["x"].to(DEV), w["gamma"].to(DEV), w["weight_offset"], w["eps"],
                what="rmsnorm_decode_16x7168")


def test_fused_workload_prefill_sampled(orc):
    w = synth.workload("rmsnorm_prefill_65536x7168", device=DEV)
    rows = torch.from_numpy(np.sort(np.random.default_rng(1).choice(65536, 2048, replace=False)))
    check_fused(orc, w["x"], w["gamma"], w["weight_offset"], w["eps"], rows_sel=rows.to(DEV),
                what="rmsnorm_prefill_65536x7168 (2048 sampled rows)")


def test_fused_grouped(orc):
    shapes = [(16, 7168), (5, 96), (33, 8192)]
    xs, gs = [], []
    for i, s in enumerate(shapes):
        x, g = synth.rmsnorm_inputs(*s, seed=40 + i, x_std=1.0, row_decades=1.0)
        xs.append(x.to(DEV))
        gs.append(g.to(DEV))
    res = mx.rmsnorm_quantize_grouped(xs, gs, [0.0, 1.0, -0.25], [1e-5, 1e-6, 1e-3])
    torch.cuda.synchronize()
    for i, (x, g, (normed, q, s)) in enumerate(zip(xs, gs, res)):
        n1, q1, s1 = mx.rmsnorm_quantize(x, g, [0.0, 1.0, -0.25][i], [1e-5, 1e-6, 1e-3][i])
        torch.cuda.synchronize()
        assert np.array_equal(host(normed.view(torch.int16)), host(n1.view(torch.int16)))
        assert np.array_equal(host(q), host(q1)) and np.array_equal(host(s), host(s1))
        q2, s2 = orc.quantize_rowwise(synth.bf16_bits(normed))
        assert_same(host(q), q2, "grouped fused q")


# -------------------------------------------------------------- dequantize --

def check_deq(orc, q, s, axis, what):
    for dtype in (torch.float32, torch.bfloat16):
        say("dequantize", what, tuple(q.shape), "axis", axis, dtype)
        out = mx.dequantize(q, s, axis, dtype)
        torch.cuda.synchronize()
        ref = orc.dequantize(host(q), host(s), axis)
        if dtype == torch.float32:
            got = host(out).astype(np.float64)
            with np.errstate(over="ignore"):
                # the exact value rounded to float32: equal unless it lies past
                # float32's range (scale bytes above 246), where it is +-inf
                ref32 = ref.astype(np.float32).astype(np.float64)
            same = (got == ref32) | (np.isnan(got) & np.isnan(ref32))
            assert same.all(), "%s: %d values differ" % (what, int((~same).sum()))
            assert (np.signbit(got[~np.isnan(ref)]) == np.signbit(ref[~np.isnan(ref)])).all()
            assert (got[np.abs(ref) < 2.0 ** 127] == ref[np.abs(ref) < 2.0 ** 127]).all()
        else:
            got = host(out.view(torch.int16)).view(np.uint16)
            want = orc.round_bf16(ref)
            nan = np.isnan(ref)
            assert_same(got[~nan], want[~nan], what + " bf16")
            assert ((got[nan] & 0x7FFF) > 0x7F80).all()


def test_dequantize_both_axes(orc):
    bits = special_values(96, 1056, seed=8)
    p = mx.quantize(dev_bits(bits), True, True)
    check_deq(orc, p.rowwise_data, p.rowwise_scale, mx.ROWWISE, "row specials")
    check_deq(orc, p.columnwise_data, p.columnwise_scale, mx.COLUMNWISE, "col specials")
    # every code under every scale byte
    q = torch.arange(256, dtype=torch.int32).to(torch.uint8).repeat(256, 1).contiguous().to(DEV)
    s = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(256, 1).repeat(1, 8).contiguous().to(DEV)
    check_deq(orc, q, s, mx.ROWWISE, "all codes x all scales")
    qc = q[:, :].T.contiguous()[:, :256]
    sc = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(1, 256).repeat(8, 1).contiguous().to(DEV)
    check_deq(orc, qc, sc, mx.COLUMNWISE, "all codes x all scales, columnwise")


def test_dequantize_weight_4096(orc):
    x = synth.workload("rowcol_4096x4096", device=DEV)["x"]
    p = mx.quantize(x, True, True)
    check_deq(orc, p.rowwise_data, p.rowwise_scale, mx.ROWWISE, "rowcol_4096x4096 row")
    check_deq(orc, p.columnwise_data, p.columnwise_scale, mx.COLUMNWISE, "rowcol_4096x4096 col")


def test_dequantize_grouped(orc):
    bits = [special_values(32 * (i + 1), 64 * (i + 1), seed=i) for i in range(3)]
    ps = [mx.quantize(dev_bits(b), True, True) for b in bits]
    outs = mx.dequantize_grouped([p.rowwise_data for p in ps] + [p.columnwise_data for p in ps],
                                 [p.rowwise_scale for p in ps] + [p.columnwise_scale for p in ps],
                                 [0, 0, 0, 1, 1, 1])
    torch.cuda.synchronize()
    for k, o in enumerate(outs):
        p = ps[k % 3]
        axis = k // 3
        q, s = (p.rowwise_data, p.rowwise_scale) if axis == 0 else (p.columnwise_data, p.columnwise_scale)
        ref = orc.dequantize(host(q), host(s), axis)
        got = host(o).astype(np.float64)
        assert ((got == ref) | (np.isnan(got) & np.isnan(ref))).all()

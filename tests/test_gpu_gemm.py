"""GPU parity of the MXFP8 matrix product against the oracle's float64 product
of the same planes.

Tolerance: the bound of tests/gemm_accuracy.py, derived from a model of the
scaled MFMA's accumulation that tests/test_gemm_accuracy_model.py pins to the
instruction with exact-input probes.  Per output it is the step-1 cut
allowance (each group of 8 products loses less than one unit 2^(E_g - 13)
per product) plus (11 n_steps + 3) 2^-24 sum_k |a_k b_k| for the float32
additions; a bf16 output adds its rounding, 2^-8 of the float32 value.  NaN
appears exactly where the oracle's product is NaN.
"""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_02_amd as mx
from tests import gemm_accuracy as acc

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print("[case]", *a, flush=True)


def host(t):
    return t.cpu().numpy()


def check_close(got, C, tol32, bf16, what):
    nan = np.isnan(C)
    assert (np.isnan(got) == nan).all(), "%s: NaN pattern differs (%d vs %d)" % (
        what, int(np.isnan(got).sum()), int(nan.sum()))
    tol = tol32 + (2.0 ** -8 * (np.abs(C) + tol32) if bf16 else 0.0)
    err = np.abs(got - C)
    bad = (err > tol) & ~nan
    assert not bad.any(), "%s: %d entries beyond tolerance, worst err/tol %.3g" % (
        what, int(bad.sum()), float((err[~nan] / np.maximum(tol[~nan], 1e-300)).max()))


def quantized(rows, cols, std, seed):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(rows, cols, generator=g) * std).to(torch.bfloat16).to(DEV)
    p = mx.quantize(x, True, False)
    return p.rowwise_data, p.rowwise_scale


def run(orc, qa, sa, qb, sb, what):
    planes = [host(t) for t in (qa, sa, qb, sb)]
    C, _ = orc.gemm(*planes)
    tol = acc.bound(*planes)
    for dtype in (torch.float32, torch.bfloat16):
        say("gemm", what, tuple(qa.shape), tuple(qb.shape), dtype)
        out = mx.gemm(qa, sa, qb, sb, dtype)
        torch.cuda.synchronize()
        got = host(out.float()).astype(np.float64)
        check_close(got, C, tol, dtype == torch.bfloat16, what)


@pytest.mark.parametrize("mnk", [(128, 128, 128), (256, 384, 512), (100, 130, 256), (1, 512, 1024),
                                 (300, 7, 128), (257, 129, 384),
                                 # ring tiles (64 x 128) and the tile128 tiles, ragged both ways
                                 (600, 900, 512), (600, 900, 384)])
def test_gemm_quantized_activation_and_weight(orc, mnk):
    M, N, K = mnk
    qa, sa = quantized(M, K, 1.0, seed=M + K)
    qb, sb = quantized(N, K, 0.05, seed=N + 7 * K)
    run(orc, qa, sa, qb, sb, "quantized")


def random_planes(rows, K, seed, lo=110, hi=145):
    g = np.random.default_rng(seed)
    q = g.integers(0, 256, (rows, K), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38                 # no NaN codes here
    s = g.integers(lo, hi, (rows, K // 32), dtype=np.uint8)
    return torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV)


@pytest.mark.parametrize("mnk", [(128, 128, 256), (192, 320, 640), (600, 900, 640)])
def test_gemm_random_planes_full_range(orc, mnk):
    M, N, K = mnk
    qa, sa = random_planes(M, K, seed=1)
    qb, sb = random_planes(N, K, seed=2)
    run(orc, qa, sa, qb, sb, "random planes")


def test_gemm_large_sampled(orc):
    M = N = K = 4096
    qa, sa = quantized(M, K, 1.0, seed=5)
    qb, sb = quantized(N, K, 0.02, seed=6)
    say("gemm 4096^3 sampled")
    out = mx.gemm(qa, sa, qb, sb, torch.float32)
    torch.cuda.synchronize()
    g = np.random.default_rng(3)
    ms, ns = g.integers(0, M, 4096), g.integers(0, N, 4096)
    ms[:64], ns[:64] = M - 1, np.arange(N - 64, N)       # include the last tile
    planes = [host(t) for t in (qa, sa, qb, sb)]
    C, _ = orc.gemm_at(*planes, ms, ns)
    got = host(out)[ms, ns].astype(np.float64)
    check_close(got, C, acc.bound_at(*planes, ms, ns), False, "4096^3 sampled")


def test_gemm_nan_elements(orc):
    qa, sa = quantized(128, 256, 1.0, seed=8)
    qb, sb = quantized(128, 256, 0.05, seed=9)
    qa[5, 17] = 0x7F                                      # NaN element in row 5
    qb[9, 200] = 0xFF                                     # NaN element in B row 9
    run(orc, qa, sa, qb, sb, "NaN elements")


def test_gemm_nan_in_short_last_group(orc):
    """K = 640 on the ring tiles: the last group's first six stages repeat
    k 448..511 with scale bytes 0.  NaN data and NaN scales in the repeated
    stage and in the live part of the short group give NaN exactly where the
    oracle's product has it."""
    qa, sa = quantized(600, 640, 1.0, seed=12)
    qb, sb = quantized(900, 640, 0.05, seed=13)
    qa[5, 460] = 0x7F                                     # NaN element in the repeated stage
    qb[9, 600] = 0xFF                                     # NaN element past k 512
    sa[4, 14] = 0xFF                                      # NaN scale of k 448..479
    sb[7, 19] = 0xFF                                      # NaN scale of the last block
    run(orc, qa, sa, qb, sb, "NaN in the short last group")


def test_gemm_nan_scale(orc):
    qa, sa = quantized(128, 256, 1.0, seed=10)
    qb, sb = quantized(128, 256, 0.05, seed=11)
    sa[3, 2] = 0xFF                                       # a NaN scale in row 3
    run(orc, qa, sa, qb, sb, "NaN scale")


@pytest.mark.parametrize("mnk", [
    # K % 512 == 0: the ring tiles, ragged M and N, one, two, three (odd: the
    # trailing group) and four 512-deep scale groups, so that the XCD pairs
    # start at different quarters of K.  256 x 256 tiles:
    (4352, 3840, 1536), (2000, 7000, 1024),
    # 128 x 256 tiles (fewer rounds over the CUs than 256 x 256):
    (4096 - 37, 4096 + 100, 512), (4096, 4096 + 256, 1024), (4096 + 1, 4096, 2048), (1000, 7100, 1024),
    # 128 x 128 tiles:
    (500, 7000, 1024), (400, 6000, 512),
    # 64 x 128 tiles (few tiles in all):
    (600, 2048, 4096), (520, 1000, 512), (520, 900, 1024),
    # 33 .. 128 rows under a wide weight (at least 144 tiles of 64 x 128), one
    # and two 64-row tiles, ragged N, a short last group:
    (64, 18432, 1024), (33, 18433, 512), (100, 9216, 512), (128, 12288, 640), (65, 9300, 1024),
    # K % 512 != 0 with K >= 512: the ring tiles' short last group, whose first
    # 2, 4 or 6 stages repeat the stage before with scales 0, on each tile size
    (4352, 3840, 640), (4096, 4096 + 256, 896), (500, 7000, 768), (520, 1000, 1152),
    (600, 2048, 11008), (2000, 1000, 4224),
    # K < 512: the register-staged 128 x 128 tiling, odd 128-deep stage counts
    (4096 - 37, 4096 + 100, 384), (4096, 4096, 128), (600, 900, 256),
    # the skinny kernel's row blocks past 128 rows with paired scale words
    # (128-row blocks of four A tiles; 64-row blocks of two) and staged ones
    (300, 2048, 11008), (129, 2752, 8320), (140, 1700, 16512), (300, 2048, 4096)])
def test_gemm_large_tiles_ragged_sampled(orc, mnk):
    """Large problems: sampled outputs, every column of the last row and every
    row of the last column."""
    M, N, K = mnk
    qa, sa = quantized(M, K, 1.0, seed=M + 3 * K)
    qb, sb = quantized(N, K, 0.05, seed=N + 5 * K)
    g = np.random.default_rng(M + N + K)
    ms = np.concatenate([g.integers(0, M, 6000), np.full(N, M - 1), np.arange(M)])
    ns = np.concatenate([g.integers(0, N, 6000), np.arange(N), np.full(M, N - 1)])
    planes = [host(t) for t in (qa, sa, qb, sb)]
    C, _ = orc.gemm_at(*planes, ms, ns)
    tol = acc.bound_at(*planes, ms, ns)
    for dtype in (torch.float32, torch.bfloat16):
        say("gemm large tiles", (M, N, K), dtype)
        out = mx.gemm(qa, sa, qb, sb, dtype)
        torch.cuda.synchronize()
        got = host(out.float())[ms, ns].astype(np.float64)
        check_close(got, C, tol, dtype == torch.bfloat16, "large tiles %s" % ((M, N, K),))


@pytest.mark.parametrize("mnk", [(1024, 1024, 512), (4352, 3840, 640), (4096, 4096 + 256, 1024), (500, 7000, 768),
                                 (520, 1000, 1152), (520, 1030, 512), (600, 2047, 640), (2000, 260, 128),
                                 (2100, 384, 256), (700, 1152, 384), (4096, 4096, 128), (1000, 4096, 384),
                                 # the skinny kernel: one, two and four A tiles per row block
                                 (129, 1000, 1152), (40, 300, 1024), (384, 1152, 384), (300, 2047, 640)])
def test_gemm_bf16_output_is_rounded_f32_output(mnk):
    """The bf16 output equals the float32 output of the same call rounded to
    nearest even, element for element.  Full ring tiles with an even N store
    bf16 through a lane exchange (whole 128-byte row segments); N not a
    multiple of 64 and tile128 tiles (rows past M skipped) take the same path;
    odd N, partial ring tiles and skinny take the other stores."""
    M, N, K = mnk
    qa, sa = quantized(M, K, 1.0, seed=M + 17 * K)
    qb, sb = quantized(N, K, 0.05, seed=N + 19 * K)
    say("gemm bf16 vs rounded f32", (M, N, K))
    f = mx.gemm(qa, sa, qb, sb, torch.float32)
    b = mx.gemm(qa, sa, qb, sb, torch.bfloat16)
    torch.cuda.synchronize()
    want = f.to(torch.bfloat16)
    bad = int((b.view(torch.int16) != want.view(torch.int16)).sum())
    assert bad == 0, "%d of %d bf16 outputs differ from the rounded float32 output" % (bad, M * N)


@pytest.mark.parametrize("mnk", [(16, 7168, 7168), (1, 4096, 4096), (32, 1000, 384), (5, 96, 128),
                                 (31, 33, 640), (17, 2048, 1152),
                                 # K = 256: two units; a wave's only unit may be the second of two
                                 (8, 64, 256), (20, 300, 256), (40, 130, 256),
                                 # scale words loaded in pairs instead of staged in LDS (more than
                                 # 32 units per wave with one or two A tiles, more than 16 with
                                 # four): one tile, one tile per 32-row block
                                 (16, 96, 16896), (40, 130, 16512),
                                 # K = 128: one unit, one active wave
                                 (33, 64, 128), (100, 200, 128),
                                 # 32 < M <= 128 with (M / 32 rounded up) x (N / 32 rounded up) <= 256
                                 # workgroups: one 32-row block per workgroup, the last one ragged
                                 (48, 2048, 1024), (33, 100, 384), (64, 4096, 128), (97, 1000, 640),
                                 (65, 2048, 256), (65, 200, 512), (100, 64, 8320),
                                 # two 32-row A tiles per workgroup (32 < M <= 64, N > 4096)
                                 (64, 7168, 7168), (40, 4200, 16512),
                                 # two A tiles per 64-row block (64 < M <= 128, 2 x N / 32 <= 256)
                                 (97, 3000, 2048), (65, 2750, 16512),
                                 # four 32-row A tiles (64 < M <= 128, N > 4096)
                                 (128, 7168, 7040), (128, 7168, 7168), (100, 4200, 8320),
                                 # wide weights just short of 144 ring tiles (128 and 142 tiles of
                                 # 64 x 128), and any width with K < 512
                                 (33, 16384, 512), (100, 9088, 512), (128, 12288, 384),
                                 # M > 128 with a narrow weight: 32-row blocks (up to 32 per strip),
                                 # 64-row blocks (65 per strip; the last of two rows), 128-row blocks
                                 (200, 1000, 640), (1000, 100, 384), (4100, 40, 256), (300, 1500, 1024),
                                 (130, 1700, 512), (500, 2000, 1024)])
def test_gemm_skinny_decode(orc, mnk):
    """A few activation rows (decode): the K-split skinny path, including K
    with fewer 128-deep units than waves and N not a multiple of 32."""
    M, N, K = mnk
    qa, sa = quantized(M, K, 1.0, seed=M + 11 * K)
    qb, sb = quantized(N, K, 0.02, seed=N + 13 * K)
    run(orc, qa, sa, qb, sb, "skinny")


@pytest.mark.parametrize("mnk", [(1000, 4096, 384), (2000, 260, 128), (1024, 1024, 512), (520, 1000, 512),
                                 (4352, 3840, 640), (16, 7168, 7168), (5, 96, 128),
                                 # the skinny kernel's row blocks: 32, 64 and 128 rows
                                 (100, 200, 512), (260, 130, 128), (129, 1000, 512), (384, 1152, 384),
                                 (300, 2048, 4096)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_gemm_output_guard_bands(mnk, dtype):
    """The product written into an [M, N] view of a larger buffer filled with
    0xA5 bytes, rows a pitch apart (N + 37: odd, N + 64: even), with padding
    before and after: every output equals the contiguous call's bit for bit,
    and no byte outside the view changes (ring tiles full and partial, the
    tile128 tiles, the skinny kernel; bf16 through the paired-row stores when
    the pitch is even)."""
    M, N, K = mnk
    qa, sa = quantized(M, K, 1.0, seed=M + 23 * K)
    qb, sb = quantized(N, K, 0.05, seed=N + 29 * K)
    ref = mx.gemm(qa, sa, qb, sb, dtype)
    bits = torch.int32 if dtype == torch.float32 else torch.int16
    fill = -0x5A5A5A5B if dtype == torch.float32 else -0x5A5B          # 0xA5A5A5A5 / 0xA5A5
    for ld in (N + 37, N + 64):
        say("gemm guard bands", mnk, dtype, ld)
        pad = 4096
        buf = torch.full((pad + M * ld + pad,), fill, dtype=bits, device=DEV)
        view = buf[pad:pad + M * ld].view(M, ld)[:, :N].view(dtype)
        out = mx.gemm(qa, sa, qb, sb, dtype, out=view)
        torch.cuda.synchronize()
        assert out.data_ptr() == view.data_ptr()
        assert torch.equal(view.view(bits), ref.view(bits)), "%s ld %d: outputs differ" % (mnk, ld)
        b = buf.cpu()
        inside = torch.zeros(b.numel(), dtype=torch.bool)
        inside[pad:pad + M * ld].view(M, ld)[:, :N] = True
        assert (b[~inside] == fill).all(), "%s ld %d: %d guard elements written" % (
            mnk, ld, int((b[~inside] != fill).sum()))

"""A seeded sweep of random shapes through every route of the library,
against the oracle: rowwise-only (flat tasks), columnwise-only (tiles, and
the narrow path for rows of any length) and both planes, bf16 and float32
input, compact and padded scale planes, the columnwise plane stored
transposed, grouped lists spanning launches, the fused RMSNorm, dequantize on
both axes, the matrix product on each of its tilings (within the
accumulation bound), and grouped products (equal to single calls)."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_02_amd as mx
from mxfp8_block_scaled_02_amd import synth
from tests import gemm_accuracy as acc
from tests import oracle_pins as P
from tests.test_gpu_parity import check_fused_out

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print("[case]", *a, flush=True)


def random_case(g):
    """(rows, cols, rowwise, columnwise) obeying the block rules."""
    kind = int(g.integers(0, 3))                  # 0 row only, 1 column only, 2 both
    if kind == 0:
        return int(g.integers(1, 300)), 32 * int(g.integers(1, 80)), True, False
    rows = 32 * int(g.integers(1, 9))
    if kind == 1:
        # columnwise only: rows of any length (not a multiple of 8: the narrow path)
        cols = 8 * int(g.integers(1, 400)) if g.random() < 0.6 else int(g.integers(1, 3200))
    else:
        cols = 32 * int(g.integers(1, 100))
    return rows, cols, kind == 2, True


def input_tensor(rows, cols, g, dtype):
    x = torch.from_numpy(g.standard_normal((rows, cols)).astype(np.float32))
    x = x * torch.from_numpy(np.exp2(g.integers(-20, 20, (rows, 1))).astype(np.float32))
    x[torch.from_numpy(g.random((rows, cols)) < 0.01)] = 0.0
    return x.to(dtype).to(DEV)


def host_bits(x):
    if x.dtype == torch.bfloat16:
        return synth.bf16_bits(x)
    return x.cpu().numpy()


@pytest.mark.parametrize("seed", range(6))
def test_random_shapes_and_routes(orc, seed):
    g = np.random.default_rng(1000 + seed)
    for case in range(12):
        rows, cols, rw, cw = random_case(g)
        dtype = torch.bfloat16 if g.random() < 0.6 else torch.float32
        padded = g.random() < 0.5
        say("seed", seed, "case", case, (rows, cols), "row" if rw else "", "col" if cw else "", dtype,
            "padded" if padded else "compact")
        x = input_tensor(rows, cols, g, dtype)
        out = None
        bufs = []
        if padded:
            sr = sc = None
            if rw:
                b, sr = mx.padded_scale_plane(rows, cols, mx.ROWWISE, int(g.integers(1, 5)),
                                              int(g.integers(1, 9)), device=DEV, fill=0xA5)
                bufs.append((b, sr))
            if cw:
                b, sc = mx.padded_scale_plane(rows, cols, mx.COLUMNWISE, int(g.integers(1, 3)),
                                              8 * int(g.integers(1, 20)), device=DEV, fill=0xA5)
                bufs.append((b, sc))
            out = mx.MXFP8Planes(None, None, sr, sc)
        p = mx.quantize(x, rw, cw, out=out)
        torch.cuda.synchronize()
        xb = host_bits(x)
        if rw:
            q, s = orc.quantize_rowwise(xb)
            assert np.array_equal(p.rowwise_data.cpu().numpy(), q), "rowwise data"
            assert np.array_equal(p.rowwise_scale.cpu().numpy(), s), "rowwise scales"
        if cw:
            q, s = orc.quantize_colwise(xb)
            assert np.array_equal(p.columnwise_data.cpu().numpy(), q), "columnwise data"
            assert np.array_equal(p.columnwise_scale.cpu().numpy(), s), "columnwise scales"
        for b, v in bufs:
            mask = torch.ones_like(b, dtype=torch.bool)
            mask[:v.shape[0], :v.shape[1]] = False
            assert bool((b[mask] == 0xA5).all()), "padding written"


@pytest.mark.parametrize("seed", range(4))
def test_random_transposed_columnwise(orc, seed):
    """The columnwise plane stored transposed, with or without the rowwise
    plane (compact or in a padded allocation), single and grouped calls."""
    g = np.random.default_rng(3000 + seed)
    for case in range(6):
        n = int(g.integers(1, 4))
        rw = g.random() < 0.6
        shapes = [(32 * int(g.integers(1, 20)), (32 if rw else 8) * int(g.integers(1, 300 if rw else 1200)))
                  for _ in range(n)]
        padded = rw and g.random() < 0.4
        dtype = torch.bfloat16 if g.random() < 0.6 else torch.float32
        say("seed", seed, "case", case, shapes, dtype, "row" if rw else "", "transposed col",
            "padded" if padded else "")
        xs = [input_tensor(r, c, g, dtype) for r, c in shapes]
        outs, bufs = [], []
        for r, c in shapes:
            sr = None
            if padded:
                b, sr = mx.padded_scale_plane(r, c, mx.ROWWISE, int(g.integers(1, 5)), int(g.integers(1, 9)),
                                              device=DEV, fill=0xA5)
                bufs.append((b, sr))
            outs.append(mx.MXFP8Planes(None, None, sr, None))
        if n == 1:
            planes = [mx.quantize(xs[0], rw, True, out=outs[0], columnwise_transposed=True)]
        else:
            planes = mx.quantize_grouped(xs, rw, True, outs=outs, columnwise_transposed=True)
        torch.cuda.synchronize()
        for x, p in zip(xs, planes):
            xb = host_bits(x)
            q, sc = orc.quantize_colwise_t(xb)
            assert np.array_equal(p.columnwise_data.cpu().numpy(), q), "transposed columnwise data"
            assert np.array_equal(p.columnwise_scale.cpu().numpy(), sc), "transposed columnwise scales"
            if rw:
                q, sr = orc.quantize_rowwise(xb)
                assert np.array_equal(p.rowwise_data.cpu().numpy(), q), "rowwise data"
                assert np.array_equal(p.rowwise_scale.cpu().numpy(), sr), "rowwise scales"
        for b, v in bufs:
            mask = torch.ones_like(b, dtype=torch.bool)
            mask[:v.shape[0], :v.shape[1]] = False
            assert bool((b[mask] == 0xA5).all()), "padding written"


@pytest.mark.parametrize("seed", range(6))
def test_random_gemm_shapes(orc, seed):
    g = np.random.default_rng(2000 + seed)
    for case in range(8):
        M = int(g.choice([int(g.integers(1, 33)), int(g.integers(33, 129)), int(g.integers(129, 400)),
                          int(g.integers(513, 1200))]))
        # a wide weight under many rows takes the ring or tile128 tiles
        N = int(g.integers(1, 700)) if M <= 512 else int(g.integers(700, 1500))
        K = 128 * int(g.integers(1, 9 if M <= 512 else 5))
        say("gemm seed", seed, "case", case, (M, N, K))
        a = input_tensor(M, K, g, torch.bfloat16)
        b = input_tensor(N, K, g, torch.bfloat16)
        pa, pb = mx.quantize(a, True, False), mx.quantize(b, True, False)
        C, mag = orc.gemm(pa.rowwise_data.cpu().numpy(), pa.rowwise_scale.cpu().numpy(),
                          pb.rowwise_data.cpu().numpy(), pb.rowwise_scale.cpu().numpy())
        got = mx.gemm(pa.rowwise_data, pa.rowwise_scale, pb.rowwise_data, pb.rowwise_scale, torch.float32)
        torch.cuda.synchronize()
        err = np.abs(got.cpu().numpy().astype(np.float64) - C)
        tol = acc.bound(*(t.cpu().numpy() for t in (pa.rowwise_data, pa.rowwise_scale,
                                                     pb.rowwise_data, pb.rowwise_scale)))
        assert (err <= tol).all(), "gemm %s beyond the accumulation bound" % ((M, N, K),)


@pytest.mark.parametrize("seed", range(3))
def test_random_grouped_gemm(orc, seed):
    """Random lists of products (token counts 0 .. 200, widths, depths, scale
    orders, output dtypes): every product run on the skinny kernel (up to 32
    rows, or 128 with K < 512) equals its single call bit for bit; the others
    (ring tiles) lie within the accumulation bound at 300 sampled outputs."""
    g = np.random.default_rng(4000 + seed)
    for case in range(3):
        n = int(g.integers(1, 45))
        dtype = torch.bfloat16 if g.random() < 0.5 else torch.float32
        specs = []
        for _ in range(n):
            K = 128 * int(g.integers(1, 20)) if g.random() < 0.9 else 16896
            M = int(g.choice([int(g.integers(0, 33)), int(g.integers(33, 129)), int(g.integers(129, 200))]))
            specs.append((M, int(g.integers(1, 600)), K))
        say("grouped gemm seed", seed, "case", case, n, "products", dtype, specs[:4])
        A, B = [], []
        for M, N, K in specs:
            order = "mfma" if K % 512 == 0 and g.random() < 0.3 else "row"
            A.append(mx.quantize(input_tensor(M, K, g, torch.bfloat16), True, False, scale_order=order))
            B.append(mx.quantize(input_tensor(N, K, g, torch.bfloat16), True, False, scale_order=order))
        got = mx.gemm_grouped([a.rowwise_data for a in A], [a.rowwise_scale for a in A],
                              [b.rowwise_data for b in B], [b.rowwise_scale for b in B], dtype)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(A, B)):
            M, N, K = specs[i]
            if M <= 32 or (M <= 128 and K < 512):
                single = mx.gemm(a.rowwise_data, a.rowwise_scale, b.rowwise_data, b.rowwise_scale, dtype)
                torch.cuda.synchronize()
                bits = torch.int32 if dtype == torch.float32 else torch.int16
                assert torch.equal(got[i].view(bits), single.view(bits)), "product %d %s" % (i, specs[i])
                continue
            hp = [t.cpu().numpy() for t in (a.rowwise_data, a.rowwise_scale, b.rowwise_data, b.rowwise_scale)]
            for j in (1, 3):
                if hp[j].ndim == 3:          # MFMA order -> compact
                    hp[j] = hp[j].transpose(1, 0, 2).reshape(hp[j].shape[1], K // 32)
            ms, ns = g.integers(0, M, 300), g.integers(0, N, 300)
            C, _ = orc.gemm_at(*hp, ms, ns)
            tol = acc.bound_at(*hp, ms, ns)
            if dtype == torch.bfloat16:
                tol = tol + 2.0 ** -8 * (np.abs(C) + tol)
            err = np.abs(got[i].float().cpu().numpy().astype(np.float64)[ms, ns] - C)
            assert (err <= tol).all(), "product %d %s beyond the accumulation bound" % (i, specs[i])


@pytest.mark.parametrize("seed", range(4))
def test_random_rmsnorm(orc, seed):
    """Rows of every RMSNorm variant (one wave, four waves, sixteen waves a row,
    rows read twice past 16384 columns), random offsets and epsilons, row
    scales over 2^-20 .. 2^20."""
    g = np.random.default_rng(3000 + seed)
    for case in range(8):
        rows = int(g.choice([int(g.integers(1, 17)), int(g.integers(17, 300)), int(g.integers(300, 1200))]))
        cols = 32 * int(g.choice([int(g.integers(1, 64)), int(g.integers(64, 300)), int(g.integers(300, 700))]))
        off = float(g.choice([0.0, 1.0, -0.25]))
        eps = float(g.choice([1e-6, 1e-5, 1e-3]))
        say("rmsnorm seed", seed, "case", case, (rows, cols), off, eps)
        x = input_tensor(rows, cols, g, torch.bfloat16)
        gamma = torch.from_numpy((1.0 + 0.1 * g.standard_normal(cols)).astype(np.float32)).to(torch.bfloat16).to(DEV)
        normed, q, s = mx.rmsnorm_quantize(x, gamma, off, eps)
        torch.cuda.synchronize()
        check_fused_out(orc, synth.bf16_bits(x), synth.bf16_bits(gamma), off, eps, synth.bf16_bits(normed),
                        q.cpu().numpy(), s.cpu().numpy(), "rmsnorm %s" % ((rows, cols),))


@pytest.mark.parametrize("seed", range(4))
def test_random_dequantize(orc, seed):
    """Random codes (NaN codes included) under random scale bytes (0xFF
    included), both axes, rows of any length on the columnwise axis, float32
    and bf16 output."""
    g = np.random.default_rng(4000 + seed)
    for case in range(10):
        axis = mx.ROWWISE if g.random() < 0.5 else mx.COLUMNWISE
        if axis == mx.ROWWISE:
            rows, cols = int(g.integers(1, 300)), 32 * int(g.integers(1, 80))
            sshape = (rows, cols // 32)
        else:
            rows = 32 * int(g.integers(1, 9))
            cols = 8 * int(g.integers(1, 400)) if g.random() < 0.6 else int(g.integers(1, 3200))
            sshape = (rows // 32, cols)
        dtype = torch.float32 if g.random() < 0.5 else torch.bfloat16
        say("dequantize seed", seed, "case", case, (rows, cols), axis, dtype)
        q = g.integers(0, 256, (rows, cols), dtype=np.uint8)
        s = g.integers(90, 170, sshape, dtype=np.uint8)
        s[g.random(sshape) < 0.02] = 0xFF
        got = mx.dequantize(torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV), axis, dtype)
        torch.cuda.synchronize()
        want = orc.dequantize(q, s, axis)
        if dtype == torch.bfloat16:
            want = P.bf16_values(orc.round_bf16(want))
        g64 = got.float().cpu().numpy().astype(np.float64)
        assert ((g64 == want) | (np.isnan(g64) & np.isnan(want))).all(), "dequantize %s" % ((rows, cols),)


@pytest.mark.parametrize("seed", range(3))
def test_random_grouped(orc, seed):
    """Lists of up to 90 tensors of random shapes (more than one launch past
    64), one request for the whole list, bf16 or float32."""
    g = np.random.default_rng(5000 + seed)
    n = int(g.integers(1, 91))
    rw, cw = [(True, False), (False, True), (True, True)][int(g.integers(0, 3))]
    dtype = torch.bfloat16 if g.random() < 0.6 else torch.float32
    shapes = []
    for _ in range(n):
        rows = 32 * int(g.integers(1, 4)) if cw else int(g.integers(1, 100))
        cols = 32 * int(g.integers(1, 33)) if rw else (8 * int(g.integers(1, 130)) if g.random() < 0.7
                                                          else int(g.integers(1, 1000)))
        shapes.append((rows, cols))
    say("grouped seed", seed, n, "tensors", "row" if rw else "", "col" if cw else "", dtype)
    xs = [input_tensor(r, c, g, dtype) for r, c in shapes]
    ps = mx.quantize_grouped(xs, rw, cw)
    torch.cuda.synchronize()
    for i, (x, p) in enumerate(zip(xs, ps)):
        xb = host_bits(x)
        if rw:
            q, s = orc.quantize_rowwise(xb)
            assert np.array_equal(p.rowwise_data.cpu().numpy(), q), "tensor %d rowwise data" % i
            assert np.array_equal(p.rowwise_scale.cpu().numpy(), s), "tensor %d rowwise scales" % i
        if cw:
            q, s = orc.quantize_colwise(xb)
            assert np.array_equal(p.columnwise_data.cpu().numpy(), q), "tensor %d columnwise data" % i
            assert np.array_equal(p.columnwise_scale.cpu().numpy(), s), "tensor %d columnwise scales" % i

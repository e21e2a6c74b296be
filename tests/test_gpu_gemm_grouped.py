"""GPU parity of the grouped matrix product (mxfp8_gemm_grouped): MoE experts,
each with its own token count, weight and output.  Every product lies within
the accumulation bound of the oracle's float64 product.  Products of up to
32 rows (up to 128 with K < 512) equal the single call on the same planes
bit for bit (the grouped launch runs the same per-tile arithmetic); the
others share ring-tile launches, whose tiles may start K at another quarter
than the single call's, so their sums may be taken in another order."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_02_amd as mx
from tests import gemm_accuracy as acc

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def say(*a):
    print("[case]", *a, flush=True)


def planes(rows, cols, std, seed, order="row"):
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(rows, cols, generator=g) * std).to(torch.bfloat16).to(DEV)
    p = mx.quantize(x, True, False, scale_order=order)
    return p.rowwise_data, p.rowwise_scale


def skinny_group(M, K):
    """The products a grouped call runs on the skinny kernel."""
    return M <= 32 or (M <= 128 and K < 512)


def same_bits(a, b):
    v = torch.int32 if a.dtype == torch.float32 else torch.int16
    return torch.equal(a.view(v), b.view(v))


def check_oracle(orc, qa, sa, qb, sb, out, what, samples=None):
    """Within the accumulation bound; samples: check that many random
    outputs (and the last row and column) instead of all."""
    hp = [t.cpu().numpy() for t in (qa, sa, qb, sb)]
    if sa.dim() == 3:            # MFMA order -> compact
        M, K = qa.shape
        hp[1] = hp[1].transpose(1, 0, 2).reshape(M, K // 32)
    if sb.dim() == 3:
        N, K = qb.shape
        hp[3] = hp[3].transpose(1, 0, 2).reshape(N, K // 32)
    got = out.float().cpu().numpy().astype(np.float64)
    if samples is not None:
        M, N = got.shape
        g = np.random.default_rng(M * 7 + N)
        ms = np.concatenate([g.integers(0, M, samples), np.full(N, M - 1), np.arange(M)])
        ns = np.concatenate([g.integers(0, N, samples), np.arange(N), np.full(M, N - 1)])
        C, _ = orc.gemm_at(*hp, ms, ns)
        tol = acc.bound_at(*hp, ms, ns)
        got = got[ms, ns]
    else:
        C, _ = orc.gemm(*hp)
        tol = acc.bound(*hp)
    if out.dtype == torch.bfloat16:
        tol = tol + 2.0 ** -8 * (np.abs(C) + tol)
    assert (np.abs(got - C) <= tol).all(), "%s: outside the accumulation bound" % what


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_moe_experts(orc, dtype):
    """12 experts, weights [N, 1024] of three widths, token counts 0 .. 300
    (up to 32: the skinny tables; above: the ring-tile tables)."""
    tokens = [0, 1, 3, 16, 31, 32, 33, 64, 100, 128, 129, 300]
    widths = [384, 520, 1000]
    K = 1024
    A = [planes(m, K, 1.0, 10 + i) for i, m in enumerate(tokens)]
    B = [planes(widths[i % 3], K, 0.05, 40 + i) for i in range(len(tokens))]
    say("grouped experts", tokens, widths, dtype)
    outs = mx.gemm_grouped([a[0] for a in A], [a[1] for a in A], [b[0] for b in B], [b[1] for b in B], dtype)
    torch.cuda.synchronize()
    for i, (a, b, o) in enumerate(zip(A, B, outs)):
        assert tuple(o.shape) == (tokens[i], widths[i % 3])
        if skinny_group(tokens[i], K):
            single = mx.gemm(a[0], a[1], b[0], b[1], dtype)
            torch.cuda.synchronize()
            assert same_bits(o, single), "expert %d (%d tokens) differs from the single call" % (i, tokens[i])
        if tokens[i]:
            check_oracle(orc, a[0], a[1], b[0], b[1], o, "expert %d" % i)


def test_many_products_both_scale_modes(orc):
    """40 skinny products (two tables of the staged mode), some with K = 16896
    (paired scale words) in between, and 10 ring-tile products: each skinny
    one equals its single call; every one is within the bound."""
    specs = [(1 + (7 * i) % 32, 64 + 32 * (i % 5), 16896 if i % 9 == 4 else 512) for i in range(40)]
    specs += [(33 + 9 * i, 96 + 40 * i, 512 if i % 2 else 1024) for i in range(10)]
    A = [planes(m, k, 1.0, 100 + i) for i, (m, n, k) in enumerate(specs)]
    B = [planes(n, k, 0.05, 200 + i) for i, (m, n, k) in enumerate(specs)]
    say("grouped 50 products", specs[:6], "...")
    outs = mx.gemm_grouped([a[0] for a in A], [a[1] for a in A], [b[0] for b in B], [b[1] for b in B])
    torch.cuda.synchronize()
    for i, (a, b, o) in enumerate(zip(A, B, outs)):
        if skinny_group(specs[i][0], specs[i][2]):
            single = mx.gemm(a[0], a[1], b[0], b[1])
            torch.cuda.synchronize()
            assert same_bits(o, single), "product %d %s differs from the single call" % (i, specs[i])
    for i in (0, 4, 13, 39) + tuple(range(40, 50)):
        check_oracle(orc, A[i][0], A[i][1], B[i][0], B[i][1], outs[i], "product %d" % i,
                     samples=2000 if specs[i][2] > 4096 else None)


def test_mfma_order_and_output_slices(orc):
    """Scales in the MFMA order, outputs written as column slices of one
    wider matrix (the experts' outputs side by side) inside a buffer of
    guard bytes: nothing outside the slices changes."""
    tokens, N, K = [5, 40, 128, 17], 256, 1536
    A = [planes(m, K, 1.0, 300 + i, "mfma") for i, m in enumerate(tokens)]
    B = [planes(N, K, 0.05, 400 + i, "mfma") for i in range(len(tokens))]
    M = max(tokens)
    pad, width = 4096, len(tokens) * N + 8
    buf = torch.full((pad + M * width + pad,), -0x5A5A5A5B, dtype=torch.int32, device=DEV)
    wide = buf[pad:pad + M * width].view(M, width).view(torch.float32)
    outs = [wide[:m, i * N:(i + 1) * N] for i, m in enumerate(tokens)]
    say("grouped mfma order, output slices", tokens)
    got = mx.gemm_grouped([a[0] for a in A], [a[1] for a in A], [b[0] for b in B], [b[1] for b in B],
                          torch.float32, outs=outs)
    torch.cuda.synchronize()
    inside = torch.zeros(buf.numel(), dtype=torch.bool, device=DEV)
    for i, m in enumerate(tokens):
        assert got[i].data_ptr() == outs[i].data_ptr()
        inside[pad:pad + M * width].view(M, width)[:m, i * N:(i + 1) * N] = True
        if skinny_group(m, K):
            single = mx.gemm(A[i][0], A[i][1], B[i][0], B[i][1])
            torch.cuda.synchronize()
            assert same_bits(got[i].contiguous(), single), "expert %d" % i
        check_oracle(orc, A[i][0], A[i][1], B[i][0], B[i][1], got[i], "expert %d" % i)
    assert bool((buf[~inside] == -0x5A5A5A5B).all()), "guard bytes written"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_prefill_experts(orc, dtype):
    """Experts of 129 .. 900 tokens share ring-tile launches, each with the
    tile its shape favours (256 x 256, 128 x 256 and 128 x 128 occur), K with
    and without a short last scale group, and one K below 512 (a single
    call)."""
    specs = [(129, 256, 512), (200, 384, 640), (256, 520, 1024), (300, 1000, 1536), (512, 256, 512),
             (640, 2048, 1024), (900, 300, 1152), (130, 130, 384), (256, 256, 2048), (384, 640, 512),
             (160, 128, 512), (170, 100, 1024)]
    A = [planes(m, k, 1.0, 500 + i) for i, (m, n, k) in enumerate(specs)]
    B = [planes(n, k, 0.05, 600 + i) for i, (m, n, k) in enumerate(specs)]
    say("grouped prefill experts", specs, dtype)
    outs = mx.gemm_grouped([a[0] for a in A], [a[1] for a in A], [b[0] for b in B], [b[1] for b in B], dtype)
    torch.cuda.synchronize()
    for i, (m, n, k) in enumerate(specs):
        assert tuple(outs[i].shape) == (m, n)
        check_oracle(orc, A[i][0], A[i][1], B[i][0], B[i][1], outs[i], "expert %s" % (specs[i],),
                     samples=None if m * n * k <= 1 << 27 else 4000)


def test_short_k_tables(orc):
    """K below 512 with 33 .. 128 rows: the skinny tables of two and four A
    tiles (equal to single calls); above 128 rows, the single call."""
    specs = [(40, 300, 384), (64, 200, 128), (100, 520, 256), (128, 64, 384), (129, 300, 256), (20, 33, 128)]
    A = [planes(m, k, 1.0, 700 + i) for i, (m, n, k) in enumerate(specs)]
    B = [planes(n, k, 0.05, 800 + i) for i, (m, n, k) in enumerate(specs)]
    say("grouped short K", specs)
    outs = mx.gemm_grouped([a[0] for a in A], [a[1] for a in A], [b[0] for b in B], [b[1] for b in B])
    torch.cuda.synchronize()
    for i, (a, b, o) in enumerate(zip(A, B, outs)):
        single = mx.gemm(a[0], a[1], b[0], b[1])
        torch.cuda.synchronize()
        assert same_bits(o, single), "product %d %s differs from the single call" % (i, specs[i])
        check_oracle(orc, a[0], a[1], b[0], b[1], o, "product %d" % i)


def test_empty_list_and_refused_product():
    assert mx.gemm_grouped([], [], [], []) == []
    qa, sa = planes(4, 256, 1.0, 1)
    qb, sb = planes(8, 128, 1.0, 2)
    with pytest.raises(ValueError):
        mx.gemm_grouped([qa], [sa], [qb], [sb])          # K 256 against 128


def test_linear_compositions(orc):
    """linear and linear_grouped equal their two explicit calls bit for bit:
    the activation quantized on the fly (in the weight's scale order), then
    the product."""
    g = torch.Generator().manual_seed(91)
    ws = [(torch.randn(n, 1024, generator=g) * 0.05).to(torch.bfloat16).to(DEV) for n in (256, 384, 512)]
    xs = [torch.randn(m, 1024, generator=g).to(torch.bfloat16).to(DEV) for m in (3, 40, 300)]
    for order in ("row", "mfma"):
        wp = [mx.quantize(w, True, False, scale_order=order) for w in ws]
        say("linear compositions", order)
        got = mx.linear_grouped(xs, wp)
        for x, w, y in zip(xs, wp, got):
            a = mx.quantize(x, True, False, scale_order=order)
            want = mx.gemm(a.rowwise_data, a.rowwise_scale, w.rowwise_data, w.rowwise_scale, torch.bfloat16)
            one = mx.linear(x, w)
            torch.cuda.synchronize()
            assert same_bits(one, want), "linear"
            if skinny_group(x.shape[0], 1024):
                assert same_bits(y, want), "linear_grouped"
            else:
                # ring tiles in the grouped launch: the same bound, not the same bits
                check_oracle(orc, a.rowwise_data, a.rowwise_scale, w.rowwise_data, w.rowwise_scale, y,
                             "linear_grouped %d rows" % x.shape[0])

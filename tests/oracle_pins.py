"""Checks that pin the CPU oracle to things other than itself.

Each check takes an ``oracle.Oracle`` and raises ``AssertionError`` on a
mismatch.  ``test_oracle_pins.py`` runs them on the oracle as built;
``test_oracle_mutants.py`` runs them on copies of the oracle with a planted
mistake and requires every copy to fail at least one check.

What the checks compare against (never the oracle's own formulas):

* hand-derived worked examples in ``golden/worked_examples.txt``;
* torch's CPU casts, which are a library special case of the element rule:
  float32 -> float8_e4m3fn rounds to nearest even (it does not saturate, so the
  value is clamped to +-448 first), and the e4m3fn / e8m0fnu -> float32 casts
  decode the formats;
* a brute-force nearest-even search over the 256 e4m3fn codes;
* properties the scale rule implies (the largest scaled magnitude of a block
  lands in [256, 512), e4m3's top binade, unless the scale is clamped);
* invariants: the half-ulp error bound, idempotence, sign symmetry, exact
  power-of-two scaling, columnwise(x) == rowwise(x^T)^T;
* for RMSNorm, an independent numpy float64 expression, closed forms for
  constant rows, and torch's float32 -> bf16 cast for the final rounding.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "worked_examples.txt")
BLOCK = 32


# ----------------------------------------------------------------- helpers --

def bf16_bits_of(values) -> np.ndarray:
    """bf16 bit patterns of float values that are exactly representable in bf16."""
    v = np.asarray(values, np.float64)
    t = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    back = t.to(torch.float64).numpy()
    same = (back == v) | (np.isnan(back) & np.isnan(v))
    assert same.all(), "value not representable in bf16: %r" % v[~same][:4]
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_values(bits) -> np.ndarray:
    """float64 values of bf16 bit patterns (bf16 is the top half of binary32)."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def torch_e4m3_bytes(v) -> np.ndarray:
    """torch's float32 -> float8_e4m3fn cast after clamping to +-448 (RNE)."""
    t = torch.from_numpy(np.asarray(v, np.float64).astype(np.float32))
    t = torch.clamp(t, -448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def e4m3_decode_table() -> np.ndarray:
    """float64 value of each of the 256 e4m3fn codes, decoded by torch."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float32).double().numpy()


def e8m0_decode(s) -> np.ndarray:
    t = torch.from_numpy(np.asarray(s, np.uint8).copy())
    return t.view(torch.float8_e8m0fnu).to(torch.float32).double().numpy()


def bruteforce_e4m3_bytes(v) -> np.ndarray:
    """Nearest e4m3fn code by exhaustive search; ties go to the even code;
    magnitudes at or beyond 448 give 448; the sign bit is always x's."""
    v = np.asarray(v, np.float64)
    table = e4m3_decode_table()
    pos_codes = np.arange(0x7F)               # 0x00 .. 0x7E: the finite magnitudes
    grid = table[pos_codes]
    a = np.minimum(np.abs(v), 448.0)
    out = np.empty(v.shape, np.uint8)
    flat_a = a.reshape(-1)
    flat_out = out.reshape(-1)
    chunk = 1 << 16
    for i in range(0, flat_a.size, chunk):
        d = np.abs(flat_a[i:i + chunk, None] - grid[None, :])
        best = d.min(axis=1, keepdims=True)
        cand = d == best
        # among equally near codes prefer the one with an even mantissa bit
        even = cand & ((pos_codes[None, :] & 1) == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
        flat_out[i:i + chunk] = pos_codes[pick]
    sign = np.signbit(v).astype(np.uint8) << 7
    return out | sign


def scaled(x_vals, s_bytes) -> np.ndarray:
    """x * 2^(127 - S), exact in float64."""
    return np.ldexp(x_vals, 127 - s_bytes.astype(np.int64))


def expected_elements(x_vals, s_bytes) -> np.ndarray:
    """Element bytes from torch's cast, given each element's scale byte."""
    nan_block = s_bytes == 0xFF
    s_safe = np.where(nan_block, 127, s_bytes)
    v = scaled(x_vals, s_safe)
    q = torch_e4m3_bytes(np.where(nan_block, 0.0, v))
    nan_q = (np.signbit(x_vals).astype(np.uint8) << 7) | 0x7F
    return np.where(nan_block, nan_q, q).astype(np.uint8)


def check_scale_property(amax, s):
    """The scale byte of a block whose largest magnitude is amax."""
    amax = np.asarray(amax, np.float64)
    s = np.asarray(s, np.int64)
    nonfinite = ~np.isfinite(amax)
    assert (s[nonfinite] == 0xFF).all(), "non-finite block must get scale 0xFF"
    zero = amax == 0
    assert (s[zero] == 0).all(), "all-zero block must get scale 0x00"
    rest = ~nonfinite & ~zero
    a, sb = amax[rest], s[rest]
    assert ((sb >= 0) & (sb <= 254)).all()
    top = np.ldexp(a, 127 - sb)
    clamped = sb == 0
    ok = np.where(clamped, top < 512, (top >= 256) & (top < 512))
    assert ok.all(), "scaled amax outside e4m3's top binade: amax=%r s=%r" % (
        a[~ok][:4], sb[~ok][:4])


# ------------------------------------------------------------------ checks --

def parse_golden():
    cases = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, vals, scale, elems, rest = [p.strip() for p in line.split("|")]
            bits = []
            for tok in vals.split():
                if tok.startswith("b:"):
                    bits.append(int(tok[2:], 16))
                else:
                    fv = float.fromhex(tok) if "0x" in tok else float(tok)
                    bits.append(int(bf16_bits_of([fv])[0]))
            cases.append((name, bits, int(scale, 16), [int(e, 16) for e in elems.split()],
                          int(rest, 16)))
    return cases


def check_golden(orc):
    cases = parse_golden()
    assert len(cases) >= 15
    for name, bits, scale, elems, rest in cases:
        x = np.zeros((1, BLOCK), np.uint16)
        x[0, :len(bits)] = bits
        q, s = orc.quantize_rowwise(x)
        want = np.full(BLOCK, rest, np.uint8)
        want[:len(elems)] = elems
        assert s[0, 0] == scale, "%s: scale %#x, expected %#x" % (name, s[0, 0], scale)
        assert (q[0] == want).all(), "%s: elements %s, expected %s" % (
            name, [hex(b) for b in q[0, :len(elems)]], [hex(b) for b in elems])
        # the same block laid down a column must give the same bytes
        qc, sc = orc.quantize_colwise(x.T.copy())
        assert sc[0, 0] == scale and (qc[:, 0] == want).all(), name + " (columnwise)"


def all_bf16_patterns() -> np.ndarray:
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def check_single_value_blocks(orc, stride: int = 1):
    """Every bf16 pattern alone in a block (the rest +0.0), at lane i % 32."""
    pats = all_bf16_patterns()[::stride]
    n = pats.size
    x = np.zeros((n, BLOCK), np.uint16)
    lane = np.arange(n) % BLOCK
    x[np.arange(n), lane] = pats
    q, s = orc.quantize_rowwise(x)
    vals = bf16_values(pats)
    check_scale_property(np.abs(vals), s[:, 0])
    want = expected_elements(vals, s[:, 0].astype(np.int64))
    got = q[np.arange(n), lane]
    bad = got != want
    assert not bad.any(), "single-value blocks: %d mismatches, first pattern %#06x -> %#04x, want %#04x" % (
        bad.sum(), pats[bad][0], got[bad][0], want[bad][0])
    # the other 31 lanes hold +0.0: 0x00, or 0x7F in a NaN-scale block
    others = np.ones((n, BLOCK), bool)
    others[np.arange(n), lane] = False
    rest_want = np.where(s[:, 0] == 0xFF, 0x7F, 0x00)[:, None]
    assert (q[others].reshape(n, BLOCK - 1) == rest_want).all(), "zero lanes"
    finite = np.isfinite(vals) & (s[:, 0] != 0xFF)
    brute = bruteforce_e4m3_bytes(scaled(vals[finite], s[finite, 0]))
    assert (brute == got[finite]).all(), "brute-force nearest-even search disagrees"


def pair_blocks(s_values=range(0, 247)):
    """Blocks [anchor, v1 .. v31]: anchor = 2^(S - 119) fixes the scale byte S,
    and v runs over every finite bf16 with |v| < 2^(S - 118)."""
    xs, ss = [], []
    for S in s_values:
        kmax = min((S + 9) << 7, 0x7F80)          # magnitude bits below 2^(S-118)
        mags = np.arange(kmax, dtype=np.uint32)
        vals = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        pad = (-vals.size) % (BLOCK - 1)
        vals = np.concatenate([vals, np.zeros(pad, np.uint16)])
        blocks = vals.reshape(-1, BLOCK - 1)
        anchor = np.uint16((S - 119 + 127) << 7) if S - 119 >= -126 else np.uint16(
            1 << (S - 119 + 133))
        col0 = np.full((blocks.shape[0], 1), anchor, np.uint16)
        xs.append(np.concatenate([col0, blocks], axis=1))
        ss.append(np.full(blocks.shape[0], S, np.int64))
    return np.concatenate(xs), np.concatenate(ss)


def check_pair_blocks(orc, s_values=range(0, 247)):
    x, s_want = pair_blocks(s_values)
    assert math.isclose(bf16_values(x[s_want == 119][:1, :1])[0, 0], 1.0)
    q, s = orc.quantize_rowwise(x)
    assert (s[:, 0] == s_want).all(), "anchor did not set the scale"
    vals = bf16_values(x)
    want = expected_elements(vals, np.repeat(s_want[:, None], BLOCK, axis=1))
    bad = q != want
    assert not bad.any(), "pair blocks: %d mismatches, first x=%#06x S=%d got %#04x want %#04x" % (
        bad.sum(), x[bad][0], np.repeat(s_want[:, None], BLOCK, 1)[bad][0], q[bad][0], want[bad][0])


def random_tensors(seed=7, rows=128, cols=256):
    """A few seeded bf16 tensors covering ordinary, wide-range and tiny values."""
    g = torch.Generator().manual_seed(seed)
    out = []
    out.append(torch.randn(rows, cols, generator=g).to(torch.bfloat16))
    out.append((torch.randn(rows, cols, generator=g) * 0.02).to(torch.bfloat16))
    mag = torch.pow(2.0, torch.empty(rows, cols).uniform_(-60, 60, generator=g))
    sign = torch.where(torch.rand(rows, cols, generator=g) < 0.5, -1.0, 1.0)
    out.append((mag * sign).to(torch.bfloat16))
    tiny = torch.randint(-(1 << 15), 1 << 15, (rows, cols), generator=g, dtype=torch.int32)
    tiny = (tiny & 0x80FF).to(torch.int16)                # bf16 subnormals and tiny normals
    out.append(tiny.view(torch.bfloat16))
    z = torch.randn(rows, cols, generator=g)
    z[:, :64] = 0.0
    z[:32, 64:96] = -0.0
    out.append(z.to(torch.bfloat16))
    return [t.view(torch.int16).numpy().view(np.uint16).copy() for t in out]


def half_ulp_bound(v):
    """Half an e4m3 ulp at the scaled value v (|v| <= 448)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6)
    return np.ldexp(0.5, (e - 3).astype(np.int64))


def check_error_bound(orc, xs):
    for x in xs:
        for axis in (0, 1):
            q, s = orc.quantize_rowwise(x) if axis == 0 else orc.quantize_colwise(x)
            s_full = (np.repeat(s, BLOCK, axis=1) if axis == 0
                      else np.repeat(s, BLOCK, axis=0)).astype(np.int64)
            vals = bf16_values(x)
            deq = orc.dequantize(q, s, axis)
            v = scaled(vals, s_full)
            sat = np.abs(v) > 448
            lim = np.ldexp(half_ulp_bound(np.where(sat, 448.0, v)), s_full - 127)
            err = np.abs(deq - vals)
            assert (err[~sat] <= lim[~sat]).all(), "error above half an e4m3 ulp"
            assert (deq[sat] == np.sign(vals[sat]) * np.ldexp(448.0, s_full[sat] - 127)).all()
            # sign of zero kept
            assert (np.signbit(deq) == np.signbit(vals)).all()


def check_idempotent(orc, xs):
    for x in xs:
        q, s = orc.quantize_rowwise(x)
        deq = orc.dequantize(q, s, 0)
        keep = (s[:, :] >= 3).all(axis=1)     # below that deq can leave bf16's range
        if not keep.any():
            continue
        back = bf16_bits_of(deq[keep])
        q2, s2 = orc.quantize_rowwise(back)
        assert (q2 == q[keep]).all() and (s2 == s[keep]).all(), "re-quantize changed bytes"


def check_sign_symmetry(orc, xs):
    for x in xs:
        q, s = orc.quantize_rowwise(x)
        qn, sn = orc.quantize_rowwise(x ^ np.uint16(0x8000))
        assert (sn == s).all() and (qn == (q ^ np.uint8(0x80))).all(), "sign symmetry"


def check_pow2_shift(orc, xs, k=5):
    for x in xs:
        vals = bf16_values(x)
        a = np.abs(vals)
        ok_rows = ((a == 0) | ((a >= 2.0 ** -100) & (a <= 2.0 ** 100))).all(axis=1)
        xr = x[ok_rows]
        if xr.shape[0] == 0:
            continue
        shifted = bf16_bits_of(np.ldexp(bf16_values(xr), k))
        q, s = orc.quantize_rowwise(xr)
        q2, s2 = orc.quantize_rowwise(shifted)
        nz = s != 0
        assert (s2[nz] == s[nz] + k).all(), "scale must move by k"
        rows_nz = nz.all(axis=1)
        assert (q2[rows_nz] == q[rows_nz]).all(), "bytes must not change under 2^k"


def check_col_is_row_of_transpose(orc, xs):
    for x in xs:
        qc, sc = orc.quantize_colwise(x)
        qr, sr = orc.quantize_rowwise(np.ascontiguousarray(x.T))
        assert (qc == qr.T).all() and (sc == sr.T).all(), "columnwise != rowwise(x^T)^T"


def check_col_t_is_row_of_transpose(orc, xs):
    """The transposed columnwise plane is, byte for byte and shape for shape,
    the rowwise plane of x^T: a plane left untransposed, or scales indexed
    the other way, fails (the tensors are not square)."""
    for x in xs:
        qt, st = orc.quantize_colwise_t(x)
        qr, sr = orc.quantize_rowwise(np.ascontiguousarray(x.T))
        assert qt.shape == qr.shape and st.shape == sr.shape, "transposed plane shapes"
        assert (qt == qr).all() and (st == sr).all(), "transposed columnwise != rowwise(x^T)"


def check_row_col_agree(orc, xs):
    for x in xs:
        vals = bf16_values(x)
        qr, sr = orc.quantize_rowwise(x)
        qc, sc = orc.quantize_colwise(x)
        dr, dc = orc.dequantize(qr, sr, 0), orc.dequantize(qc, sc, 1)
        ok = np.isfinite(vals)
        br = np.ldexp(half_ulp_bound(np.minimum(np.abs(scaled(vals, np.repeat(sr, 32, 1).astype(np.int64))), 448)),
                      np.repeat(sr, 32, 1).astype(np.int64) - 127)
        bc = np.ldexp(half_ulp_bound(np.minimum(np.abs(scaled(vals, np.repeat(sc, 32, 0).astype(np.int64))), 448)),
                      np.repeat(sc, 32, 0).astype(np.int64) - 127)
        sat = (np.abs(scaled(vals, np.repeat(sr, 32, 1).astype(np.int64))) > 448) | (
            np.abs(scaled(vals, np.repeat(sc, 32, 0).astype(np.int64))) > 448)
        m = ok & ~sat
        assert (np.abs(dr - dc)[m] <= (br + bc)[m]).all(), "row and column planes disagree"


def check_dequant_tables(orc):
    # every e4m3 code at scale 1 (byte 127) decodes as torch decodes it
    q = np.arange(256, dtype=np.uint32).astype(np.uint8).reshape(8, 32)
    s = np.full((8, 1), 127, np.uint8)
    got = orc.dequantize(q, s, 0).reshape(-1)
    want = e4m3_decode_table()
    assert ((got == want) | (np.isnan(got) & np.isnan(want))).all(), "e4m3 decode"
    # every scale byte, applied to the code of 1.0 (0x38)
    sb = np.arange(256, dtype=np.uint32).astype(np.uint8)
    q1 = np.full((256, 32), 0x38, np.uint8)
    got = orc.dequantize(q1, sb.reshape(256, 1), 0)[:, 0]
    want = e8m0_decode(sb)
    assert ((got == want) | (np.isnan(got) & np.isnan(want))).all(), "e8m0 decode"
    # columnwise indexing: scale row i covers rows 32i .. 32i+31
    qc = np.full((64, 3), 0x38, np.uint8)
    scb = np.array([[120, 121, 122], [130, 131, 132]], np.uint8)
    got = orc.dequantize(qc, scb, 1)
    assert (got[:32] == np.ldexp(1.0, scb[0].astype(np.int64) - 127)).all()
    assert (got[32:] == np.ldexp(1.0, scb[1].astype(np.int64) - 127)).all()


def check_round_bf16(orc, n=200000, seed=3):
    g = np.random.default_rng(seed)
    bits = g.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.round_bf16(f.astype(np.float64))
    assert (got == want).all(), "bf16 rounding of float32 values"
    # exact ties in float64 that float32 cannot hold
    ties = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8) * 2.0 ** -130])
    got = orc.round_bf16(ties)
    assert list(got) == [0x3F80, 0x3F82, bf16_bits_of([-2.0 ** -130])[0]]
    assert orc.round_bf16(np.array([np.nan]))[0] & 0x7FFF == 0x7FC0


def check_rmsnorm(orc, seed=11):
    g = torch.Generator().manual_seed(seed)
    rows, cols = 16, 96
    x = (torch.randn(rows, cols, generator=g) *
         torch.pow(10.0, torch.empty(rows, 1).uniform_(-3, 2, generator=g))).to(torch.bfloat16)
    gamma = (torch.randn(cols, generator=g) * 0.1 + 1).to(torch.bfloat16)
    xb = x.view(torch.int16).numpy().view(np.uint16).copy()
    gb = gamma.view(torch.int16).numpy().view(np.uint16).copy()
    for off, eps in ((1.0, 1e-6), (0.0, 1e-5), (-0.5, 1e-2)):
        y = orc.rmsnorm_f64(xb, gb, off, eps)
        xv, gv = bf16_values(xb), bf16_values(gb)
        eps32 = float(np.float32(eps))
        ref = xv / np.sqrt(np.mean(xv * xv, axis=1, keepdims=True) + eps32) * (gv + off)
        assert np.allclose(y, ref, rtol=1e-12, atol=0), "RMSNorm formula"
        normed = orc.rmsnorm(xb, gb, off, eps)
        assert (normed == orc.round_bf16(y)).all(), "normed is y rounded once"
        n2, q, s = orc.rmsnorm_quantize(xb, gb, off, eps)
        q2, s2 = orc.quantize_rowwise(normed)
        assert (n2 == normed).all() and (q == q2).all() and (s == s2).all()
    # gamma = 1, offset 0: textbook RMSNorm, mean(y^2) = ms / (ms + eps)
    ones = bf16_bits_of(np.ones(cols))
    y = orc.rmsnorm_f64(xb, ones, 0.0, 1e-5)
    ms = np.mean(bf16_values(xb) ** 2, axis=1)
    eps32 = float(np.float32(1e-5))
    assert np.allclose(np.mean(y * y, axis=1), ms / (ms + eps32), rtol=1e-12)
    # constant row c: y = c / sqrt(c^2 + eps) * w
    c = bf16_bits_of(np.full((1, cols), -1.5))
    y = orc.rmsnorm_f64(c, gb, 0.25, 1e-2)
    eps32 = float(np.float32(1e-2))
    want = -1.5 / math.sqrt(2.25 + eps32) * (bf16_values(gb) + 0.25)
    assert np.allclose(y[0], want, rtol=1e-14)


def check_rmsnorm_range(orc, seed=13):
    """RMSNorm over bf16's whole range.  With eps = 0 the formula is invariant
    under x -> 2^k x, and in binary floating point that holds bit for bit as
    long as nothing overflows or underflows: squares, their sum, the mean and
    the square root all scale by exact powers of two.  So rows at 2^-125 ..
    2^126 must give the very same doubles as the row at 2^0, and a row of
    bf16 subnormals m 2^-133 the same as m 2^-100.  The rows the formula
    leaves undefined follow IEEE arithmetic: 0/0 is NaN, x * 0 is 0 for finite
    x and NaN for an infinity."""
    g = np.random.default_rng(seed)
    cols = 224
    gam = torch.from_numpy((1.0 + 0.1 * g.standard_normal(cols)).astype(np.float32))
    gb = bf16_bits_of(gam.to(torch.bfloat16).double().numpy())
    # |x| in [0.5, 2): every 2^k multiple for k in -125 .. 126 is a normal bf16
    mag = g.uniform(0.5, 1.99, cols) * np.where(g.random(cols) < 0.5, -1.0, 1.0)
    mag = torch.from_numpy(mag.astype(np.float32)).to(torch.bfloat16).double().numpy()
    base = bf16_bits_of(mag)[None, :]
    want = orc.rmsnorm_f64(base, gb, 0.5, 0.0)
    for k in (-125, -100, -60, 1, 60, 100, 126):
        xk = bf16_bits_of(bf16_values(base) * 2.0 ** k)
        assert (bf16_values(xk) == bf16_values(base) * 2.0 ** k).all()
        got = orc.rmsnorm_f64(xk, gb, 0.5, 0.0)
        assert (got == want).all(), "RMSNorm not scale invariant at 2^%d" % k
        assert (orc.rmsnorm(xk, gb, 0.5, 0.0) == orc.round_bf16(want)).all()
    # subnormal row m 2^-133 against its normal twin m 2^-100 (m = 1 .. 127)
    m = g.integers(1, 128, cols) * np.where(g.random(cols) < 0.5, -1.0, 1.0)
    sub = bf16_bits_of(m * 2.0 ** -133)[None, :]
    assert ((sub & 0x7F80) == 0).all() and (bf16_values(sub) == m * 2.0 ** -133).all()
    twin = bf16_bits_of(m * 2.0 ** -100)[None, :]
    assert (orc.rmsnorm_f64(sub, gb, 0.0, 0.0) == orc.rmsnorm_f64(twin, gb, 0.0, 0.0)).all()
    # a positive eps 2^29 times below the mean square (rows at 2^-60) moves
    # rstd by about 2^-30; against rows at 2^-100 it dominates: then
    # y = x / sqrt(mean(x^2) + eps) * w with eps the larger term
    eps = float(np.float32(1e-45))                   # the smallest float32, 2^-149
    assert eps == 2.0 ** -149
    x60 = bf16_bits_of(bf16_values(base) * 2.0 ** -60)
    assert np.allclose(orc.rmsnorm_f64(x60, gb, 0.5, eps), want, rtol=2.0 ** -28, atol=0)
    assert not (orc.rmsnorm_f64(x60, gb, 0.5, eps) == want).all()
    x100 = bf16_bits_of(bf16_values(base) * 2.0 ** -100)
    w = bf16_values(gb) + 0.5
    ms = np.mean(bf16_values(x100) ** 2)
    ref = bf16_values(x100)[0] / math.sqrt(ms + eps) * w
    assert np.allclose(orc.rmsnorm_f64(x100, gb, 0.5, eps)[0], ref, rtol=1e-14, atol=0)
    # zero rows: NaN with eps = 0, signed zeros with eps > 0
    z = np.zeros((1, cols), np.uint16)
    z[0, ::3] = 0x8000
    assert np.isnan(orc.rmsnorm_f64(z, gb, 0.5, 0.0)).all()
    assert ((orc.rmsnorm(z, gb, 0.5, 0.0) & 0x7FFF) == 0x7FC0).all()
    y0 = orc.rmsnorm_f64(z, gb, 0.5, 1e-5)
    assert (y0 == 0).all() and (np.signbit(y0) == (z == 0x8000) ^ (w < 0)).all()
    # infinities: rstd = 0, so finite values give signed zeros and the
    # infinities 0 * inf = NaN; a NaN anywhere makes the whole row NaN
    inf_row = base.copy()
    inf_row[0, 7], inf_row[0, 100] = 0x7F80, 0xFF80
    y = orc.rmsnorm_f64(inf_row, gb, 0.5, 1e-5)
    assert np.isnan(y[0, [7, 100]]).all()
    rest = np.ones(cols, bool)
    rest[[7, 100]] = False
    assert (y[0, rest] == 0).all()
    assert (np.signbit(y[0, rest]) == (np.signbit(bf16_values(base)[0, rest]) ^ (w[rest] < 0))).all()
    nan_row = base.copy()
    nan_row[0, 50] = 0x7FC1
    assert np.isnan(orc.rmsnorm_f64(nan_row, gb, 0.5, 1e-5)).all()
    # the quantized plane of a NaN row: every block NaN
    _, q, s = orc.rmsnorm_quantize(nan_row, gb, 0.5, 1e-5)
    assert (s == 0xFF).all() and ((q & 0x7F) == 0x7F).all()


def f32_blocks(seed=17, nblocks=4096):
    """float32 blocks: random values over a wide exponent range, plus blocks of
    exact e4m3 ties and ties +- 1 float32 ulp under an anchor that fixes the
    scale byte, so the rounding sees every bit of float32 precision."""
    g = np.random.default_rng(seed)
    mant = g.uniform(1.0, 2.0, (nblocks, 32))
    expo = g.integers(-140, 120, (nblocks, 1)) + g.integers(-20, 1, (nblocks, 32))
    sign = np.where(g.random((nblocks, 32)) < 0.5, -1.0, 1.0)
    x = (sign * np.ldexp(mant, expo)).astype(np.float32)
    x[g.random((nblocks, 32)) < 0.02] = 0.0
    # ties: midpoints of the e4m3 grid at scale 2^0 (anchor 256 -> S = 127)
    grid = e4m3_decode_table()[:0x7F]
    mids = (grid[:-1] + grid[1:]) / 2
    t = []
    for m in mids:
        m32 = np.float32(m)
        t += [m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9))]
    t = np.array(t, np.float32)
    pad = (-t.size) % 31
    t = np.concatenate([t, np.zeros(pad, np.float32)]).reshape(-1, 31)
    anchor = np.full((t.shape[0], 1), 256.0, np.float32)
    ties = np.concatenate([anchor, t], axis=1)
    neg = -ties
    # the same ties at a large and a tiny scale (exact power-of-two shifts)
    big = np.ldexp(ties.astype(np.float64), 60).astype(np.float32)
    tiny = np.ldexp(ties.astype(np.float64), -100).astype(np.float32)
    return np.concatenate([x, ties, neg, big, tiny]).astype(np.float32)


def check_f32_input(orc):
    x = f32_blocks()
    q, s = orc.quantize_rowwise(x)
    vals = x.astype(np.float64)
    check_scale_property(np.abs(vals).max(axis=1), s[:, 0])
    want = expected_elements(vals, np.repeat(s.astype(np.int64), 32, axis=1))
    bad = q != want
    assert not bad.any(), "float32 rowwise: %d mismatches, first x=%r S=%d got %#x want %#x" % (
        bad.sum(), vals[bad][0], np.repeat(s, 32, 1)[bad][0], q[bad][0], want[bad][0])
    xt = np.ascontiguousarray(x.T)
    qc, sc = orc.quantize_colwise(xt)
    assert (qc == q.T).all() and (sc == s.T).all(), "float32 columnwise != rowwise of transpose"
    # a bf16-representable float32 tensor quantizes exactly like its bf16 bits
    b = random_tensors(seed=5, rows=64, cols=64)[2]
    qb, sb = orc.quantize_rowwise(b)
    qf, sf = orc.quantize_rowwise(bf16_values(b).astype(np.float32))
    assert (qb == qf).all() and (sb == sf).all(), "float32 and bf16 paths disagree"


def check_gemm(orc, seed=23):
    """The MXFP8 product against numpy's float64 matmul of the dequantized
    planes, a brute-force loop on a tiny case, and exact special cases."""
    g = torch.Generator().manual_seed(seed)
    M, N, K = 48, 40, 160
    a = (torch.randn(M, K, generator=g) * torch.pow(2.0, torch.randint(-6, 7, (M, 1), generator=g))).to(torch.bfloat16)
    b = (torch.randn(N, K, generator=g) * 0.05).to(torch.bfloat16)
    qa, sa = orc.quantize_rowwise(a.view(torch.int16).numpy().view(np.uint16))
    qb, sb = orc.quantize_rowwise(b.view(torch.int16).numpy().view(np.uint16))
    C, mag = orc.gemm(qa, sa, qb, sb)
    da, db = orc.dequantize(qa, sa, 0), orc.dequantize(qb, sb, 0)
    ref = da @ db.T
    assert np.allclose(C, ref, rtol=1e-12, atol=1e-300), "product against numpy"
    assert np.allclose(mag, np.abs(da) @ np.abs(db).T, rtol=1e-12), "abs sums"
    # brute force on a corner
    for m in (0, 7, M - 1):
        for n in (0, 13, N - 1):
            s_ = sum(da[m, k] * db[n, k] for k in range(K))
            assert math.isclose(C[m, n], s_, rel_tol=1e-12, abs_tol=1e-300)
    # positions
    ms, ns = np.array([0, 5, M - 1]), np.array([N - 1, 3, 0])
    v, _ = orc.gemm_at(qa, sa, qb, sb, ms, ns)
    assert (v == C[ms, ns]).all()
    # exact special case: one-hot blocks with known scales
    q1 = np.zeros((2, 64), np.uint8); s1 = np.full((2, 2), 127, np.uint8)
    q1[0, 3] = 0x38; q1[1, 40] = 0x40          # 1.0 at k = 3; 2.0 at k = 40
    s1[1, 1] = 130                              # second block of row 1 scaled by 2^3
    q2 = np.zeros((3, 64), np.uint8); s2 = np.full((3, 2), 127, np.uint8)
    q2[0, 3] = 0x38; q2[1, 40] = 0xC4; q2[2, 3] = 0x7E   # 1.0, -3.0 (0xC4), 448
    s2[1, 1] = 126
    C1, _ = orc.gemm(q1, s1, q2, s2)
    want = np.array([[1.0, 0.0, 448.0], [0.0, 2.0 * 8 * -3.0 * 0.5, 0.0]])
    assert (C1 == want).all(), C1


QUICK_CHECKS = [
    ("golden", check_golden),
    ("single_value_blocks", lambda o: check_single_value_blocks(o, stride=1)),
    ("pair_blocks_sample", lambda o: check_pair_blocks(o, s_values=[0, 1, 2, 3, 8, 9, 119, 127, 200, 246])),
    ("dequant_tables", check_dequant_tables),
    ("round_bf16", check_round_bf16),
    ("rmsnorm", check_rmsnorm),
    ("rmsnorm_range", check_rmsnorm_range),
    ("col_is_row_of_transpose", lambda o: check_col_is_row_of_transpose(o, random_tensors(rows=64, cols=64))),
    ("error_bound", lambda o: check_error_bound(o, random_tensors(rows=64, cols=64))),
    ("f32_input", check_f32_input),
    ("gemm", check_gemm),
]

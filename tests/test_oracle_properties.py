"""Property tests of the CPU oracle (no GPU): hypothesis draws tensor shapes
(multiples of 32) and contents with injected zeros, signed zeros, bf16
subnormals, outliers, whole zero blocks and, in one test, NaN/Inf.  Every
example is checked against what the format fixes independently of the
oracle's code: each block's scale puts its largest magnitude in e4m3's top
binade (or is 0x00 / 0xFF), every element byte equals torch's clamped
float8_e4m3fn cast of x * 2^(127 - S), and the invariants (error bound, sign
symmetry, columnwise = rowwise of the transpose, planes agree)."""
import numpy as np
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

from tests import oracle_pins as P

SETTINGS = settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])


def to_bf16_bits(values) -> np.ndarray:
    """bf16 patterns of float values, rounded to nearest even."""
    t = torch.from_numpy(np.asarray(values, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


@st.composite
def tensors(draw, nonfinite=False):
    rows = 32 * draw(st.integers(1, 4))
    cols = 32 * draw(st.integers(1, 4))
    g = np.random.default_rng(draw(st.integers(0, 2 ** 32 - 1)))
    # rows of different magnitudes, 2^-40 .. 2^40
    x = g.standard_normal((rows, cols)) * np.ldexp(1.0, g.integers(-40, 41, (rows, 1)))
    bits = to_bf16_bits(x)
    u = g.random((rows, cols))
    bits[u < 0.05] = 0x0000                                        # +0
    bits[(u >= 0.05) & (u < 0.08)] = 0x8000                        # -0
    sub = (g.integers(1, 128, (rows, cols)) | (g.integers(0, 2, (rows, cols)) << 15)).astype(np.uint16)
    m = (u >= 0.08) & (u < 0.12)
    bits[m] = sub[m]                                               # bf16 subnormals
    out = to_bf16_bits(P.bf16_values(bits) * 1000.0)
    m = (u >= 0.12) & (u < 0.13)
    bits[m] = out[m]                                               # outliers x1000
    if draw(st.booleans()):                                        # a whole zero block
        r, c = 32 * g.integers(0, rows // 32), 32 * g.integers(0, cols // 32)
        bits[r:r + 32, c:c + 32] = 0
    if nonfinite:
        specials = np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC1], np.uint16)   # +-Inf, +-NaN
        k = draw(st.integers(1, 6))
        bits[g.integers(0, rows, k), g.integers(0, cols, k)] = specials[g.integers(0, 4, k)]
    return bits


def check_plane(x_bits, q, s, axis):
    vals = P.bf16_values(x_bits)
    rows, cols = vals.shape
    blocks = (vals.reshape(rows, cols // 32, 32) if axis == 0
              else vals.reshape(rows // 32, 32, cols).transpose(0, 2, 1))
    with np.errstate(invalid="ignore"):
        amax = np.max(np.abs(blocks), axis=2)
    P.check_scale_property(amax, s)
    s_full = (np.repeat(s, 32, axis=1) if axis == 0 else np.repeat(s, 32, axis=0)).astype(np.int64)
    assert (q == P.expected_elements(vals, s_full)).all(), "element bytes differ from the clamped cast"


@SETTINGS
@given(tensors())
def test_planes_against_scale_rule_and_torch_cast(orc, x):
    qr, sr = orc.quantize_rowwise(x)
    qc, sc = orc.quantize_colwise(x)
    check_plane(x, qr, sr, 0)
    check_plane(x, qc, sc, 1)


@SETTINGS
@given(tensors(nonfinite=True))
def test_nonfinite_blocks(orc, x):
    qr, sr = orc.quantize_rowwise(x)
    qc, sc = orc.quantize_colwise(x)
    check_plane(x, qr, sr, 0)
    check_plane(x, qc, sc, 1)
    # the other blocks do not notice: clearing the non-finite elements
    # changes only the blocks that held them
    vals = P.bf16_values(x)
    bad = ~np.isfinite(vals)
    x2 = np.where(bad, np.uint16(0), x)
    qr2, sr2 = orc.quantize_rowwise(x2)
    bad_blocks = bad.reshape(bad.shape[0], -1, 32).any(axis=2)
    assert (sr2[~bad_blocks] == sr[~bad_blocks]).all()
    keep = ~np.repeat(bad_blocks, 32, axis=1)
    assert (qr2[keep] == qr[keep]).all()


@SETTINGS
@given(tensors())
def test_invariants(orc, x):
    xs = [x]
    P.check_error_bound(orc, xs)
    P.check_sign_symmetry(orc, xs)
    P.check_col_is_row_of_transpose(orc, xs)
    P.check_row_col_agree(orc, xs)

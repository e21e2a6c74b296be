"""The C ABI library without a GPU: it loads, exports every function that
include/mxfp8.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import mxfp8_block_scaled_02_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp8.h")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_NO_OUTPUT, ERR_ARG, ERR_HIP = range(7)
A = 0x10000   # aligned fake device addresses: never dereferenced, every call fails checks
B = 0x20000
C = 0x30000
D = 0x40000
MIS = 0x10008


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxfp8_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mx.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    return mx.lib()


def test_every_declared_function_is_exported(L):
    names = declared_functions()
    assert len(names) == 12, names
    for n in names:
        assert hasattr(L, n), "missing export " + n


def test_version_and_status_strings(L):
    assert L.mxfp8_abi_version() == 4
    for code in range(7):
        assert L.mxfp8_status_string(code)
    assert b"unknown" in L.mxfp8_status_string(99)


def test_quantize_argument_checks(L):
    q = L.mxfp8_quantize
    assert q(A, -1, 32, B, C, None, None, None) == ERR_SHAPE
    assert q(A, 4, 48, B, C, None, None, None) == ERR_SHAPE          # partial row block
    assert q(A, 48, 32, None, None, B, C, None) == ERR_SHAPE         # partial column block
    assert q(A, 40, 36, None, None, B, C, None) == ERR_SHAPE         # narrow columnwise: rows % 32 still
    assert q(A, 4, 32, B, None, None, None, None) == ERR_NULL        # half a plane
    assert q(A, 32, 32, None, None, None, C, None) == ERR_NULL
    assert q(None, 4, 32, B, C, None, None, None) == ERR_NULL
    assert q(A, 4, 32, None, None, None, None, None) == ERR_NO_OUTPUT
    assert q(MIS, 4, 32, B, C, None, None, None) == ERR_ALIGN
    assert q(A, 4, 32, B, C + 1, None, None, None) == ERR_ALIGN
    assert q(A, 1 << 40, 1 << 40, B, C, None, None, None) == ERR_SHAPE   # overflow
    # more tasks than one launch carries (2^45 elements, about 2^31 tasks)
    assert q(A, 1 << 23, 1 << 22, B, C, None, None, None) == ERR_SHAPE
    # empty tensors are a no-op, whatever the pointers
    assert q(None, 0, 32, None, None, None, None, None) == OK
    assert q(None, 5, 0, None, None, None, None, None) == OK


def test_rmsnorm_argument_checks(L):
    r = L.mxfp8_rmsnorm_quantize
    assert r(A, B, 0.0, 1e-6, 4, 48, C, D, A, None) == ERR_SHAPE
    assert r(A, None, 0.0, 1e-6, 4, 32, C, D, A, None) == ERR_NULL
    assert r(A, B, 0.0, float("nan"), 4, 32, C, D, A, None) == ERR_ARG
    assert r(A, B, 0.0, -1.0, 4, 32, C, D, A, None) == ERR_ARG
    assert r(A, B, 0.0, 1e-6, 4, 32, C, D, MIS, None) == ERR_ALIGN
    assert r(A, B, 0.0, 1e-6, 1 << 31, 32, C, D, A, None) == ERR_SHAPE
    assert r(None, None, 0.0, 1e-6, 0, 32, None, None, None, None) == OK


def test_dequantize_argument_checks(L):
    d = L.mxfp8_dequantize
    assert d(A, B, 4, 32, 2, C, 0, None) == ERR_ARG           # axis
    assert d(A, B, 4, 32, 0, C, 7, None) == ERR_ARG           # out dtype
    assert d(A, B, 4, 48, 0, C, 0, None) == ERR_SHAPE
    assert d(A, B, 40, 32, 1, C, 0, None) == ERR_SHAPE
    assert d(A, None, 4, 32, 0, C, 0, None) == ERR_NULL
    assert d(A, B, 4, 32, 0, MIS, 1, None) == ERR_ALIGN
    assert d(None, None, 0, 0, 1, None, 1, None) == OK


def test_gemm_argument_checks(L):
    g = L.mxfp8_gemm
    assert g(A, B, C, D, 4, 4, 96, 0, 0, A, 0, 0, None) == ERR_SHAPE       # K % 128
    assert g(A, B, C, D, 4, 4, 0, 0, 0, A, 0, 0, None) == ERR_SHAPE
    assert g(A, B, C, D, -1, 4, 128, 0, 0, A, 0, 0, None) == ERR_SHAPE
    assert g(A, None, C, D, 4, 4, 128, 0, 0, A, 0, 0, None) == ERR_NULL
    assert g(A, B, C, D, 4, 4, 128, 0, 0, MIS, 0, 0, None) == ERR_ALIGN
    assert g(A, B, C, D, 4, 4, 128, 0, 0, A, 0, 5, None) == ERR_ARG
    assert g(None, None, None, None, 0, 4, 128, 0, 0, None, 0, 0, None) == OK
    # scale pitches: at least K/32 bytes, a multiple of 4, not negative
    assert g(A, B, C, D, 4, 4, 256, 4, 0, A, 0, 0, None) == ERR_SHAPE
    assert g(A, B, C, D, 4, 4, 256, 0, 6, A, 0, 0, None) == ERR_SHAPE
    assert g(A, B, C, D, 4, 4, 256, 10, 0, A, 0, 0, None) == ERR_ALIGN
    assert g(A, B, C, D, 4, 4, 256, -8, 0, A, 0, 0, None) == ERR_SHAPE
    # output pitch: 0 or at least N
    assert g(A, B, C, D, 4, 4, 256, 0, 0, A, 3, 0, None) == ERR_SHAPE
    assert g(A, B, C, D, 4, 4, 256, 0, 0, A, -4, 0, None) == ERR_SHAPE
    assert g(A, B, C, D, 4, 4, 256, 0, 0, A, 1 << 62, 0, None) == ERR_SHAPE
    # more output tiles than 32-bit grid and tile indices hold
    assert g(A, B, C, D, 1, 1 << 40, 128, 0, 0, A, 0, 0, None) == ERR_SHAPE
    assert g(A, B, C, D, 1 << 21, 1 << 21, 128, 0, 0, A, 0, 0, None) == ERR_SHAPE


def test_grouped_checks_every_descriptor_first(L):
    good = mx._QuantDesc(A, 4, 32, B, C, None, None)
    bad = mx._QuantDesc(A, 4, 48, B, C, None, None)
    arr = (mx._QuantDesc * 3)(good, good, bad)
    # the bad third entry fails the call before the good ones are launched
    assert L.mxfp8_quantize_grouped(arr, 3, None) == ERR_SHAPE
    assert L.mxfp8_quantize_grouped(arr, -1, None) == ERR_ARG
    assert L.mxfp8_quantize_grouped(None, 2, None) == ERR_NULL
    assert L.mxfp8_quantize_grouped(None, 0, None) == OK
    n = (mx._NormDesc * 1)(mx._NormDesc(A, B, 0.0, float("inf"), 4, 32, C, D, A))
    assert L.mxfp8_rmsnorm_quantize_grouped(n, 1, None) == ERR_ARG
    dq = (mx._DeqDesc * 1)(mx._DeqDesc(A, B, 32, 40, 1, MIS))
    assert L.mxfp8_dequantize_grouped(dq, 1, 0, None) == ERR_ALIGN
    dq = (mx._DeqDesc * 1)(mx._DeqDesc(A, B, 40, 36, 1, C))        # narrow columnwise: rows % 32 still
    assert L.mxfp8_dequantize_grouped(dq, 1, 0, None) == ERR_SHAPE


def test_scale_pitch_checks(L):
    Q = mx._QuantDesc
    def quant(*d):
        return L.mxfp8_quantize_grouped((Q * 1)(Q(*d)), 1, None)
    assert quant(A, 4, 64, B, C, None, None, 1, 0) == ERR_SHAPE           # rowwise pitch < 2
    assert quant(A, 4, 64, B, C, None, None, -4, 0) == ERR_SHAPE
    assert quant(A, 32, 64, None, None, B, C, 0, 60) == ERR_SHAPE        # columnwise pitch < 64
    assert quant(A, 32, 64, None, None, B, C, 0, 68) == ERR_ALIGN        # not a multiple of 8
    assert quant(A, 32, 60, None, None, B, C, 0, 58) == ERR_SHAPE        # narrow columnwise: pitch < cols
    # a pitch whose last scale row would overflow 64-bit offsets
    assert quant(A, 1 << 20, 64, B, C, None, None, 1 << 60, 0) == ERR_SHAPE
    assert quant(A, 1 << 20, 64, None, None, B, C, 0, 1 << 60) == ERR_SHAPE
    # rowwise only, pitched: the flat block index must fit 32 bits
    assert quant(A, 1 << 30, 1024, B, C, None, None, 64, 0) == ERR_SHAPE
    assert L.mxfp8_quantize_f32_grouped((Q * 1)(Q(A, 4, 64, B, C, None, None, 1, 0)), 1, None) == ERR_SHAPE
    N = mx._NormDesc
    assert L.mxfp8_rmsnorm_quantize_grouped((N * 1)(N(A, B, 0.0, 1e-6, 4, 64, C, D, A, 1)), 1, None) == ERR_SHAPE
    assert L.mxfp8_rmsnorm_quantize_grouped((N * 1)(N(A, B, 0.0, 1e-6, 1 << 20, 64, C, D, A, 1 << 60)), 1,
                                            None) == ERR_SHAPE
    Dq = mx._DeqDesc
    assert L.mxfp8_dequantize_grouped((Dq * 1)(Dq(A, B, 4, 64, 0, C, 1)), 1, 0, None) == ERR_SHAPE
    assert L.mxfp8_dequantize_grouped((Dq * 1)(Dq(A, B, 32, 64, 1, C, 72 + 4)), 1, 0, None) == ERR_ALIGN
    assert L.mxfp8_dequantize_grouped((Dq * 1)(Dq(A, B, 32, 64, 1, C, 32)), 1, 0, None) == ERR_SHAPE
    assert L.mxfp8_dequantize_grouped((Dq * 1)(Dq(A, B, 1 << 20, 64, 0, C, 1 << 60)), 1, 0, None) == ERR_SHAPE


def test_grouped_gemm_checks(L):
    """Every product of a grouped call is checked before the first launch,
    with mxfp8_gemm's rules.  Only rejected calls are made here (no GPU)."""
    G = mx._GemmDesc
    def grouped(*ds, dtype=0):
        return L.mxfp8_gemm_grouped((G * len(ds))(*[G(*d) for d in ds]), len(ds), dtype, None)
    good = (A, B, C, D, 4, 4, 128, 0, 0, A, 0)
    assert grouped(good, (A, B, C, D, 4, 4, 96, 0, 0, A, 0)) == ERR_SHAPE     # K % 128, after a valid one
    assert grouped(good, (A, B, C, None, 4, 4, 128, 0, 0, A, 0)) == ERR_NULL
    assert grouped(good, (A, B, C, D, 4, 4, 128, 0, 0, MIS, 0)) == ERR_ALIGN
    assert grouped(good, (A, B, C, D, 4, 4, 128, 0, 0, A, 3)) == ERR_SHAPE     # out pitch < N
    assert grouped(good, (A, B, C, D, 4, 4, 256, -1, 0, A, 0)) == ERR_SHAPE    # MFMA order needs K % 512
    assert grouped(good, dtype=7) == ERR_ARG
    assert L.mxfp8_gemm_grouped(None, 2, 0, None) == ERR_NULL
    assert L.mxfp8_gemm_grouped(None, -1, 0, None) == ERR_ARG
    assert L.mxfp8_gemm_grouped(None, 0, 0, None) == OK
    assert grouped((A, B, C, D, 0, 4, 96, 0, 0, None, 0)) == OK               # M == 0: a no-op, as in mxfp8_gemm
    assert grouped((A, B, C, D, -1, 4, 128, 0, 0, A, 0)) == ERR_SHAPE


def test_transposed_columnwise_checks(L):
    """Columnwise pitch MXFP8_COLUMNWISE_T (-2): rows % 32 and cols % 8, for
    bf16 and float32 input; every descriptor of a mixed list is checked, and every
    tensor's task count too, before the first launch.  Only rejected calls
    are made here (no GPU)."""
    Q, T = mx._QuantDesc, -2
    def quant(*ds):
        return L.mxfp8_quantize_grouped((Q * len(ds))(*[Q(*d) for d in ds]), len(ds), None)
    assert quant((A, 32, 12, None, None, B, C, 0, T)) == ERR_SHAPE       # cols % 8
    assert quant((A, 48, 64, None, None, B, C, 0, T)) == ERR_SHAPE       # rows % 32
    assert quant((A, 32, 48, D, A, B, C, 0, T)) == ERR_SHAPE             # rowwise plane: cols % 32
    assert quant((A, 32, 64, None, None, B, C, 0, -3)) == ERR_SHAPE      # no other sentinel
    assert quant((A, 32, 64, None, None, B, MIS, 0, T)) == ERR_ALIGN
    assert quant((A, 32, 64, None, None, B, None, 0, T)) == ERR_NULL
    # more tasks than one launch carries: refused before the valid first
    # tensor is launched (a launch would fail here with ERR_HIP)
    assert quant((A, 32, 64, B, C, None, None, 0, 0),
                 (A, 1 << 24, 1 << 23, None, None, B, C, 0, T)) == ERR_SHAPE
    f32 = lambda *ds: L.mxfp8_quantize_f32_grouped((Q * len(ds))(*[Q(*d) for d in ds]), len(ds), None)
    assert f32((A, 32, 12, None, None, B, C, 0, T)) == ERR_SHAPE
    assert f32((A, 32, 64, B, C, None, None, 0, 0),
               (A, 1 << 24, 1 << 22, None, None, B, C, 0, T)) == ERR_SHAPE


def test_mfma_scale_order_checks(L):
    """Pitch MXFP8_SCALES_MFMA (-1): rowwise scales only, whole 512-column
    groups; any other negative pitch stays an error.  Only rejected calls are
    made here (no GPU)."""
    Q, N, Dq, M = mx._QuantDesc, mx._NormDesc, mx._DeqDesc, -1
    def quant(*d):
        return L.mxfp8_quantize_grouped((Q * 1)(Q(*d)), 1, None)
    assert quant(A, 4, 64, B, C, None, None, M, 0) == ERR_SHAPE          # cols % 512
    assert quant(A, 4, 1536, B, C, None, None, -2, 0) == ERR_SHAPE       # no other sentinel
    assert quant(A, 32, 512, None, None, B, C, 0, M) == ERR_SHAPE        # columnwise scales
    assert quant(A, 1 << 30, 1024, B, C, None, None, M, 0) == ERR_SHAPE  # flat block index > 2^32
    assert quant(A, 4, 512, B, MIS, None, None, M, 0) == ERR_ALIGN       # still checked
    assert L.mxfp8_rmsnorm_quantize_grouped((N * 1)(N(A, B, 0.0, 1e-6, 4, 96, C, D, A, M)), 1, None) == ERR_SHAPE
    assert L.mxfp8_dequantize_grouped((Dq * 1)(Dq(A, B, 4, 96, 0, C, M)), 1, 0, None) == ERR_SHAPE
    assert L.mxfp8_dequantize_grouped((Dq * 1)(Dq(A, B, 32, 512, 1, C, M)), 1, 0, None) == ERR_SHAPE
    g = L.mxfp8_gemm
    assert g(A, B, C, D, 4, 4, 256, M, 0, A, 0, 0, None) == ERR_SHAPE       # K % 512
    assert g(A, B, C, D, 4, 4, 640, 0, M, A, 0, 0, None) == ERR_SHAPE
    assert g(A, B, C, D, 4, 4, 512, -2, 0, A, 0, 0, None) == ERR_SHAPE
    assert g(A, B, C, D, 4, 4, 512, M, M, MIS, 0, 0, None) == ERR_ALIGN     # reaches the later checks


def test_mfma_scale_plane_shapes():
    """Host-side: a contiguous [cols/512, rows, 16] tensor is a plane in the
    MFMA order; other 3-D shapes and non-contiguous ones are rejected."""
    import torch
    assert mx.mfma_scale_shape(100, 1536) == (3, 100, 16)
    with pytest.raises(ValueError):
        mx.mfma_scale_shape(100, 1056)
    t = torch.zeros(3, 100, 16, dtype=torch.uint8)
    assert mx._scale_pitch(t, (100, 48), t.device, "s")[1] == -1
    with pytest.raises(ValueError):
        mx._scale_pitch(t, (100, 32), t.device, "s")
    with pytest.raises(ValueError):
        mx._scale_pitch(torch.zeros(100, 3, 16, dtype=torch.uint8).transpose(0, 1), (100, 48), t.device, "s")
    s, pitch = mx._scale_pitch(None, (100, 48), t.device, "s", mfma=True)
    assert tuple(s.shape) == (3, 100, 16) and pitch == -1
    with pytest.raises(ValueError):
        mx._mfma("cols")


def test_padded_scale_plane_views():
    """Host-side helper: the plane is the top-left view of a padded buffer and
    its row stride is what the library receives as the pitch."""
    import torch
    buf, view = mx.padded_scale_plane(100, 1056, mx.ROWWISE, 128, 4, device="cpu", fill=0xA5)
    assert tuple(buf.shape) == (128, 36) and tuple(view.shape) == (100, 33)
    assert view.stride() == (36, 1) and view.data_ptr() == buf.data_ptr()
    assert mx._scale_pitch(view, (100, 33), view.device, "s")[1] == 36
    buf, view = mx.padded_scale_plane(64, 1056, mx.COLUMNWISE, 4, 128, device="cpu")
    assert tuple(buf.shape) == (4, 1152) and tuple(view.shape) == (2, 1056)
    assert mx._scale_pitch(view, (2, 1056), view.device, "s")[1] == 1152
    compact = torch.zeros(2, 1056, dtype=torch.uint8)
    assert mx._scale_pitch(compact, (2, 1056), compact.device, "s")[1] == 0
    with pytest.raises(ValueError):
        mx._scale_pitch(compact.t(), (1056, 2), compact.device, "s")


def test_descriptor_layout_matches_header():
    # the ctypes mirrors must have the C structs' sizes (x86-64 ABI)
    assert ctypes.sizeof(mx._QuantDesc) == 72
    assert ctypes.sizeof(mx._NormDesc) == 72
    assert ctypes.sizeof(mx._DeqDesc) == 56


def test_python_layer_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        mx.quantize(torch.zeros(4, 32, dtype=torch.bfloat16))

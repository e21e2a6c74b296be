"""MXFP8 block quantization on AMD MI355X (gfx950): Python binding.

This module only marshals arguments to ``libmxfp8.so`` (C ABI in
``include/mxfp8.h``); every step of the computation runs in its HIP kernels.
torch provides device memory and the current stream.  If the library has not
been built the first call raises ``RuntimeError``; there is no fallback.

Format: blocks of 32 bf16 values share one float8_e8m0fnu scale byte and each
value becomes one float8_e4m3fn byte (Megatron-Core quantized_dbuffer page,
"Data"; Mojo DistributedAllGatherRMSNormQuantMXFP8 page, "Parameters").
Planes are returned in rowwise-data-first order (quantized_dbuffer page,
QuantizedDBuffer.planes): rowwise data, columnwise data, rowwise scale,
columnwise scale, all as ``torch.uint8`` tensors; ``as_fp8`` views them with
the float8 dtypes.  Tensors with more than two dims are flattened into rows
(Mojo page, "Parameters", rank).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import NamedTuple, Optional, Sequence

import torch

__all__ = [
    "MXFP8Planes", "quantize", "rmsnorm_quantize", "dequantize", "quantize_grouped",
    "rmsnorm_quantize_grouped", "dequantize_grouped", "gemm", "gemm_grouped", "linear", "linear_grouped", "as_fp8",
    "library_path", "lib",
    "BLOCK", "ROWWISE", "COLUMNWISE", "MFMA_GROUP", "mfma_scale_shape",
]

BLOCK = 32
ABI_VERSION = 4
ROWWISE, COLUMNWISE = 0, 1
_OUT_F32, _OUT_BF16 = 0, 1
# Rowwise scales in the MFMA order (see include/mxfp8.h, "Scale pitches"):
# a [rows, cols] tensor's scales as a uint8 tensor [cols / 512, rows, 16],
# passed to the library with the pitch MXFP8_SCALES_MFMA.
MFMA_GROUP = 512
_SCALES_MFMA = -1
# The columnwise plane stored transposed (include/mxfp8.h, MXFP8_COLUMNWISE_T):
# data [cols, rows], scales [cols, rows/32], a rowwise plane of x^T.
_COLUMNWISE_T = -2
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmxfp8.so")
_lib = None

_STATUS = {0: "MXFP8_OK", 1: "MXFP8_ERR_NULL", 2: "MXFP8_ERR_SHAPE", 3: "MXFP8_ERR_ALIGN",
           4: "MXFP8_ERR_NO_OUTPUT", 5: "MXFP8_ERR_ARG", 6: "MXFP8_ERR_HIP"}


class _QuantDesc(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("q_row", ctypes.c_void_p), ("s_row", ctypes.c_void_p),
                ("q_col", ctypes.c_void_p), ("s_col", ctypes.c_void_p),
                ("s_row_pitch", ctypes.c_int64), ("s_col_pitch", ctypes.c_int64)]


class _NormDesc(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("gamma", ctypes.c_void_p),
                ("weight_offset", ctypes.c_float), ("eps", ctypes.c_float),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("normed", ctypes.c_void_p), ("q_row", ctypes.c_void_p),
                ("s_row", ctypes.c_void_p), ("s_row_pitch", ctypes.c_int64)]


class _GemmDesc(ctypes.Structure):
    _fields_ = [("qa", ctypes.c_void_p), ("sa", ctypes.c_void_p), ("qb", ctypes.c_void_p),
                ("sb", ctypes.c_void_p), ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("sa_pitch", ctypes.c_int64), ("sb_pitch", ctypes.c_int64), ("out", ctypes.c_void_p),
                ("out_pitch", ctypes.c_int64)]


class _DeqDesc(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("s", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("axis", ctypes.c_int), ("out", ctypes.c_void_p),
                ("s_pitch", ctypes.c_int64)]


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded C library (raises RuntimeError if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libmxfp8.so is not built; run `python -m "
                           "mxfp8_block_scaled_02_amd.build` (or __graft_entry__.build())")
    L = ctypes.CDLL(_LIB_PATH)
    p, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    L.mxfp8_abi_version.argtypes, L.mxfp8_abi_version.restype = [], ctypes.c_int
    if L.mxfp8_abi_version() != ABI_VERSION:
        raise RuntimeError("libmxfp8.so has ABI version %d, this binding expects %d; rebuild it"
                           % (L.mxfp8_abi_version(), ABI_VERSION))
    L.mxfp8_status_string.argtypes, L.mxfp8_status_string.restype = [ctypes.c_int], ctypes.c_char_p
    L.mxfp8_quantize.argtypes = [p, i64, i64, p, p, p, p, p]
    L.mxfp8_rmsnorm_quantize.argtypes = [p, p, f32, f32, i64, i64, p, p, p, p]
    L.mxfp8_dequantize.argtypes = [p, p, i64, i64, ctypes.c_int, p, ctypes.c_int, p]
    L.mxfp8_quantize_grouped.argtypes = [ctypes.POINTER(_QuantDesc), i32, p]
    L.mxfp8_quantize_f32.argtypes = [p, i64, i64, p, p, p, p, p]
    L.mxfp8_quantize_f32_grouped.argtypes = [ctypes.POINTER(_QuantDesc), i32, p]
    L.mxfp8_rmsnorm_quantize_grouped.argtypes = [ctypes.POINTER(_NormDesc), i32, p]
    L.mxfp8_gemm.argtypes = [p, p, p, p, i64, i64, i64, i64, i64, p, i64, ctypes.c_int, p]
    L.mxfp8_dequantize_grouped.argtypes = [ctypes.POINTER(_DeqDesc), i32, ctypes.c_int, p]
    L.mxfp8_gemm_grouped.argtypes = [ctypes.POINTER(_GemmDesc), i32, ctypes.c_int, p]
    for name in ("mxfp8_quantize", "mxfp8_rmsnorm_quantize", "mxfp8_dequantize",
                 "mxfp8_quantize_grouped", "mxfp8_rmsnorm_quantize_grouped",
                 "mxfp8_dequantize_grouped", "mxfp8_quantize_f32", "mxfp8_quantize_f32_grouped",
                 "mxfp8_gemm", "mxfp8_gemm_grouped"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int) -> None:
    if status == 0:
        return
    msg = "%s: %s" % (_STATUS.get(status, status), lib().mxfp8_status_string(status).decode())
    if status == 6:
        raise RuntimeError(msg)
    raise ValueError(msg)


class MXFP8Planes(NamedTuple):
    """Physical planes of one MXFP8 tensor in rowwise-data-first order; a plane
    that was not requested is None."""
    rowwise_data: Optional[torch.Tensor]
    columnwise_data: Optional[torch.Tensor]
    rowwise_scale: Optional[torch.Tensor]
    columnwise_scale: Optional[torch.Tensor]


def as_fp8(planes: MXFP8Planes) -> MXFP8Planes:
    """The same storage viewed as float8_e4m3fn data and float8_e8m0fnu scales."""
    def v(t, dt):
        return None if t is None else t.view(dt)
    return MXFP8Planes(v(planes.rowwise_data, torch.float8_e4m3fn),
                       v(planes.columnwise_data, torch.float8_e4m3fn),
                       v(planes.rowwise_scale, torch.float8_e8m0fnu),
                       v(planes.columnwise_scale, torch.float8_e8m0fnu))


# float8 views of the byte planes (as_fp8) are accepted where bytes are
_BYTE_ALIASES = {torch.float8_e4m3fn: torch.uint8, torch.float8_e8m0fnu: torch.uint8}


def _bytes(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.uint8) if t.dtype in _BYTE_ALIASES else t


def _as2d(x: torch.Tensor, name: str, dtype=torch.bfloat16, device=None) -> torch.Tensor:
    if dtype == torch.uint8:
        x = _bytes(x)
    if x.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, x.dtype))
    if not x.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if device is not None and x.device != device:
        raise ValueError("%s must be on %s, got %s" % (name, device, x.device))
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if x.dim() == 0:
        raise ValueError("%s must have at least one dimension" % name)
    if x.dim() == 1:
        return x.view(1, -1)
    return x.reshape(-1, x.shape[-1]) if x.dim() > 2 else x


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


# torch's own C entry points for the current device and raw stream, when this
# build has them (a few microseconds less per call than the public wrappers)
_get_device = getattr(torch._C, "_cuda_getDevice", None)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device) -> int:
    if _raw_stream is not None and device.index is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _on(device):
    """The device context for a call: none when the device is already current
    (stream 0 would name the current device's null stream)."""
    if _get_device is not None and device.index is not None and _get_device() == device.index:
        return contextlib.nullcontext()
    return torch.cuda.device(device)


def _out(t, shape, dtype, device, name):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if dtype == torch.uint8:
        t = _bytes(t)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %s tensor of shape %s on %s" % (name, dtype, tuple(shape), device))
    return t


def mfma_scale_shape(rows: int, cols: int) -> tuple:
    """Shape of the rowwise scales of a [rows, cols] tensor in the MFMA order:
    (cols / 512, rows, 16); block b of row r is element [b // 16, r, b % 16]."""
    if cols % MFMA_GROUP:
        raise ValueError("the MFMA scale order needs cols %% %d == 0, got %d" % (MFMA_GROUP, cols))
    return (cols // MFMA_GROUP, rows, MFMA_GROUP // BLOCK)


def _scale_pitch(t, shape, device, name, allocate=True, mfma=False):
    """A scale plane [rows, width] as (tensor, pitch).  The tensor may be a view
    of a larger, padded allocation whose rows are stride(0) bytes apart: that
    stride goes to the library as the plane's pitch (0 when compact).  A
    contiguous 3-D tensor [width / 16, rows, 16] (or mfma=True when the plane
    is allocated here) is a rowwise plane in the MFMA order."""
    if t is None:
        if not allocate:
            raise ValueError("%s is required" % name)
        if mfma:
            return torch.empty(mfma_scale_shape(shape[0], shape[1] * BLOCK), dtype=torch.uint8,
                               device=device), _SCALES_MFMA
        return torch.empty(shape, dtype=torch.uint8, device=device), 0
    t = _bytes(t)
    if t.dim() == 3:
        want = mfma_scale_shape(shape[0], shape[1] * BLOCK)
        if t.dtype != torch.uint8 or tuple(t.shape) != want or t.device != device or not t.is_contiguous():
            raise ValueError("%s in the MFMA order must be a contiguous uint8 tensor of shape %s on %s"
                             % (name, want, device))
        return t, _SCALES_MFMA
    if t.dtype != torch.uint8 or tuple(t.shape) != tuple(shape) or t.device != device:
        raise ValueError("%s must be a uint8 tensor of shape %s on %s" % (name, tuple(shape), device))
    if t.dim() != 2 or (shape[1] > 1 and t.stride(1) != 1) or (
            shape[0] > 1 and shape[1] > 0 and t.stride(0) < shape[1]):
        raise ValueError("%s must have unit column stride and a row stride >= its width" % name)
    pitch = t.stride(0) if shape[0] > 1 else shape[1]
    return t, (0 if pitch == shape[1] else pitch)


def _mfma(scale_order: str) -> bool:
    if scale_order not in ("row", "mfma"):
        raise ValueError("scale_order must be 'row' or 'mfma', got %r" % (scale_order,))
    return scale_order == "mfma"


def padded_scale_plane(rows: int, cols: int, axis: int = 0, row_multiple: int = 1,
                       col_multiple: int = 1, device=None, fill: int = 0):
    """A scale plane for a [rows, cols] tensor inside a padded allocation.

    The plane ([rows, cols/32] rowwise, [rows/32, cols] columnwise) is the
    top-left view of a uint8 buffer whose shape is rounded up to multiples of
    (row_multiple, col_multiple) and filled with `fill`; pass the view as an
    output (or input) plane and the kernels use the buffer's row pitch
    directly.  Returns (buffer, view)."""
    shape = (rows, cols // BLOCK) if axis == ROWWISE else (rows // BLOCK, cols)
    r = -(-shape[0] // row_multiple) * row_multiple
    c = -(-shape[1] // col_multiple) * col_multiple
    buf = torch.full((r, c), fill, dtype=torch.uint8, device=device)
    return buf, buf[:shape[0], :shape[1]]


def _quant_desc(x, rowwise, columnwise, out, mfma=False, transposed=False):
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("x must be bfloat16 or float32, got %s" % x.dtype)
    x2 = _as2d(x, "x", x.dtype)
    rows, cols = x2.shape
    o = out or MXFP8Planes(None, None, None, None)
    dev = x.device
    qr = _out(o.rowwise_data, (rows, cols), torch.uint8, dev, "rowwise_data") if rowwise else None
    sr, pr = (_scale_pitch(o.rowwise_scale, (rows, cols // BLOCK), dev, "rowwise_scale", mfma=mfma)
              if rowwise else (None, 0))
    if columnwise and transposed:
        qc = _out(o.columnwise_data, (cols, rows), torch.uint8, dev, "columnwise_data")
        sc = _out(o.columnwise_scale, (cols, rows // BLOCK), torch.uint8, dev, "columnwise_scale")
        pc = _COLUMNWISE_T
    else:
        qc = _out(o.columnwise_data, (rows, cols), torch.uint8, dev, "columnwise_data") if columnwise else None
        sc, pc = (_scale_pitch(o.columnwise_scale, (rows // BLOCK, cols), dev, "columnwise_scale")
                  if columnwise else (None, 0))
    if pc == _SCALES_MFMA:
        raise ValueError("columnwise_scale: the MFMA order is for rowwise scales only")
    d = _QuantDesc(_ptr(x2), rows, cols, _ptr(qr), _ptr(sr), _ptr(qc), _ptr(sc), pr, pc)
    return d, MXFP8Planes(qr, qc, sr, sc)


def quantize(x: torch.Tensor, rowwise: bool = True, columnwise: bool = False,
             out: Optional[MXFP8Planes] = None, scale_order: str = "row",
             columnwise_transposed: bool = False) -> MXFP8Planes:
    """Quantize x [rows, cols] (bf16, or a float32 master weight) into the
    requested planes in one launch.

    ``out`` supplies persistent plane buffers that are overwritten in place
    (Megatron-Core quantization.utils page, quantize_params_to_mxfp8).
    ``scale_order="mfma"`` writes the rowwise scales in the MFMA order
    (cols % 512 == 0), which ``gemm`` and ``dequantize`` accept as they are.
    ``columnwise_transposed=True`` (cols % 8 == 0) stores the
    columnwise plane transposed, data [cols, rows] and scales
    [cols, rows/32]: a rowwise plane of x^T, which ``gemm`` takes as an
    operand contracting over the rows of x."""
    d, planes = _quant_desc(x, rowwise, columnwise, out, _mfma(scale_order), columnwise_transposed)
    with _on(x.device):
        if d.s_row_pitch or d.s_col_pitch:
            # padded scale planes: a one-entry grouped call carries the pitches
            fn = lib().mxfp8_quantize_grouped if x.dtype == torch.bfloat16 else lib().mxfp8_quantize_f32_grouped
            _check(fn((_QuantDesc * 1)(d), 1, _stream(x.device)))
        else:
            fn = lib().mxfp8_quantize if x.dtype == torch.bfloat16 else lib().mxfp8_quantize_f32
            _check(fn(d.x, d.rows, d.cols, d.q_row, d.s_row, d.q_col, d.s_col, _stream(x.device)))
    return planes


def quantize_grouped(xs: Sequence[torch.Tensor], rowwise: bool = True, columnwise: bool = False,
                     outs: Optional[Sequence[MXFP8Planes]] = None, scale_order: str = "row",
                     columnwise_transposed: bool = False) -> list:
    """Quantize a list of tensors of any shapes (all bf16 or all float32) in one
    launch (``columnwise_transposed``: see ``quantize``)."""
    mfma = _mfma(scale_order)
    if not xs:
        return []
    dev, dt = xs[0].device, xs[0].dtype
    descs, planes = [], []
    for i, x in enumerate(xs):
        if x.device != dev or x.dtype != dt:
            raise ValueError("all tensors must share one device and one dtype")
        d, p = _quant_desc(x, rowwise, columnwise, outs[i] if outs else None, mfma, columnwise_transposed)
        descs.append(d)
        planes.append(p)
    arr = (_QuantDesc * len(descs))(*descs)
    fn = lib().mxfp8_quantize_grouped if dt == torch.bfloat16 else lib().mxfp8_quantize_f32_grouped
    with _on(dev):
        _check(fn(arr, len(descs), _stream(dev)))
    return planes


def _norm_desc(x, gamma, weight_offset, eps, out, mfma=False):
    x2 = _as2d(x, "x")
    rows, cols = x2.shape
    g = _as2d(gamma, "gamma", device=x.device)
    if g.numel() != cols:
        raise ValueError("gamma must have %d elements" % cols)
    dev = x.device
    o = out or (None, None, None)
    normed = _out(o[0], (rows, cols), torch.bfloat16, dev, "normed")
    q = _out(o[1], (rows, cols), torch.uint8, dev, "q")
    s, pitch = _scale_pitch(o[2], (rows, cols // BLOCK), dev, "s", mfma=mfma)
    d = _NormDesc(_ptr(x2), _ptr(g), float(weight_offset), float(eps), rows, cols,
                  _ptr(normed), _ptr(q), _ptr(s), pitch)
    return d, (normed, q, s)


def rmsnorm_quantize(x: torch.Tensor, gamma: torch.Tensor, weight_offset: float = 0.0,
                     eps: float = 1e-6, out=None, scale_order: str = "row"):
    """RMSNorm (sum of squares and rstd in float64, the products in float32)
    rounded once to bf16, then its rowwise MXFP8 plane.

    Returns (normed bf16 [rows, cols], data uint8 [rows, cols], scales uint8
    [rows, cols/32], or [cols/512, rows, 16] with ``scale_order="mfma"``); the
    bytes equal ``quantize(normed)``."""
    d, res = _norm_desc(x, gamma, weight_offset, eps, out, _mfma(scale_order))
    with _on(x.device):
        if d.s_row_pitch:
            _check(lib().mxfp8_rmsnorm_quantize_grouped((_NormDesc * 1)(d), 1, _stream(x.device)))
        else:
            _check(lib().mxfp8_rmsnorm_quantize(d.x, d.gamma, d.weight_offset, d.eps, d.rows,
                                                d.cols, d.normed, d.q_row, d.s_row,
                                                _stream(x.device)))
    return res


def rmsnorm_quantize_grouped(xs, gammas, weight_offsets, epss, outs=None, scale_order: str = "row") -> list:
    """Fused RMSNorm + rowwise quantize over a list of tensors in one launch."""
    mfma = _mfma(scale_order)
    if not xs:
        return []
    dev = xs[0].device
    descs, res = [], []
    for i, x in enumerate(xs):
        if x.device != dev:
            raise ValueError("all tensors must be on one device")
        d, r = _norm_desc(x, gammas[i], weight_offsets[i], epss[i], outs[i] if outs else None, mfma)
        descs.append(d)
        res.append(r)
    arr = (_NormDesc * len(descs))(*descs)
    with _on(dev):
        _check(lib().mxfp8_rmsnorm_quantize_grouped(arr, len(descs), _stream(dev)))
    return res


def _deq_desc(q, s, axis, dtype, out):
    q2 = _as2d(q, "q", torch.uint8)
    rows, cols = q2.shape
    want = (rows, cols // BLOCK) if axis == ROWWISE else (rows // BLOCK, cols)
    if not s.is_cuda:
        raise ValueError("s must be a GPU tensor")
    s2, pitch = _scale_pitch(s, want, q.device, "s", allocate=False)
    if pitch == _SCALES_MFMA and axis != ROWWISE:
        raise ValueError("s: the MFMA order is for rowwise scales only")
    o = _out(out, (rows, cols), dtype, q.device, "out")
    return _DeqDesc(_ptr(q2), _ptr(s2), rows, cols, int(axis), _ptr(o), pitch), o


def _out_code(dtype):
    if dtype == torch.float32:
        return _OUT_F32
    if dtype == torch.bfloat16:
        return _OUT_BF16
    raise ValueError("dequantize output must be float32 or bfloat16")


def dequantize(q: torch.Tensor, s: torch.Tensor, axis: int = ROWWISE,
               dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None):
    """Values of one plane, e4m3(q) * 2^(s - 127), as float32 or bf16."""
    code = _out_code(dtype)
    d, o = _deq_desc(q, s, axis, dtype, out)
    with _on(q.device):
        if d.s_pitch:
            _check(lib().mxfp8_dequantize_grouped((_DeqDesc * 1)(d), 1, code, _stream(q.device)))
        else:
            _check(lib().mxfp8_dequantize(d.q, d.s, d.rows, d.cols, d.axis, d.out, code,
                                          _stream(q.device)))
    return o


def dequantize_grouped(qs, ss, axes, dtype=torch.float32, outs=None) -> list:
    if not qs:
        return []
    code = _out_code(dtype)
    dev = qs[0].device
    descs, res = [], []
    for i, q in enumerate(qs):
        d, o = _deq_desc(q, ss[i], axes[i], dtype, outs[i] if outs else None)
        descs.append(d)
        res.append(o)
    arr = (_DeqDesc * len(descs))(*descs)
    with _on(dev):
        _check(lib().mxfp8_dequantize_grouped(arr, len(descs), code, _stream(dev)))
    return res


def gemm(qa: torch.Tensor, sa: torch.Tensor, qb: torch.Tensor, sb: torch.Tensor,
         dtype: torch.dtype = torch.float32, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[M, N] = A . B^T from rowwise planes A = (qa [M, K], sa [M, K/32]) and
    B = (qb [N, K], sb [N, K/32]) (quantization.utils page, mm_mxfp8: a
    quantized activation times a pre-quantized weight [out, in]).  Either
    scale plane may be in the MFMA order ([K/512, rows, 16], K % 512 == 0).
    ``out`` may be a view whose rows lie further apart than N (a column slice
    of a wider matrix); only its [M, N] elements are written."""
    d, o = _gemm_desc(qa, sa, qb, sb, dtype, out)
    with _on(qa.device):
        _check(lib().mxfp8_gemm(d.qa, d.sa, d.qb, d.sb, d.M, d.N, d.K, d.sa_pitch, d.sb_pitch, d.out, d.out_pitch,
                                _out_code(dtype), _stream(qa.device)))
    return o


def gemm_grouped(qas: Sequence[torch.Tensor], sas: Sequence[torch.Tensor], qbs: Sequence[torch.Tensor],
                 sbs: Sequence[torch.Tensor], dtype: torch.dtype = torch.float32,
                 outs: Optional[Sequence[Optional[torch.Tensor]]] = None) -> list:
    """n independent products outs[i] = A_i . B_i^T in as few launches as the
    library can (MoE experts with a few tokens each share launches); each
    result equals gemm's for the same operands.  Arguments as for gemm, one
    per product, all on one device."""
    n = len(qas)
    if not (len(sas) == len(qbs) == len(sbs) == n) or (outs is not None and len(outs) != n):
        raise ValueError("gemm_grouped: one qa, sa, qb, sb (and out) per product")
    if n == 0:
        return []
    dev = qas[0].device
    descs, res = [], []
    for i in range(n):
        if qas[i].device != dev:
            raise ValueError("gemm_grouped: all products must be on one device")
        d, o = _gemm_desc(qas[i], sas[i], qbs[i], sbs[i], dtype, outs[i] if outs is not None else None)
        descs.append(d)
        res.append(o)
    arr = (_GemmDesc * n)(*descs)
    with _on(dev):
        _check(lib().mxfp8_gemm_grouped(arr, n, _out_code(dtype), _stream(dev)))
    return res


def linear(x: torch.Tensor, w: MXFP8Planes, dtype: torch.dtype = torch.bfloat16,
           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x [M, K] (bf16) times a pre-quantized weight w [N, K] (its rowwise plane)
    transposed: the activation is quantized on the fly, then multiplied
    (quantization.utils page, mm_mxfp8).  Two library calls; the activation's
    scales take the weight's scale order."""
    order = "mfma" if w.rowwise_scale.dim() == 3 else "row"
    a = quantize(x, True, False, scale_order=order)
    return gemm(a.rowwise_data, a.rowwise_scale, w.rowwise_data, w.rowwise_scale, dtype, out=out)


def linear_grouped(xs: Sequence[torch.Tensor], ws: Sequence[MXFP8Planes], dtype: torch.dtype = torch.bfloat16,
                   outs: Optional[Sequence[Optional[torch.Tensor]]] = None) -> list:
    """The experts of an MoE layer: xs[i] [M_i, K_i] (bf16, any M_i) times the
    pre-quantized weight ws[i] [N_i, K_i]: one grouped quantize of the
    activations, then one grouped product."""
    if len(xs) != len(ws):
        raise ValueError("linear_grouped: one weight per activation")
    if not xs:
        return []
    orders = {"mfma" if w.rowwise_scale.dim() == 3 else "row" for w in ws}
    if len(orders) != 1:
        raise ValueError("linear_grouped: the weights' scales must share one order")
    a = quantize_grouped(xs, True, False, scale_order=orders.pop())
    return gemm_grouped([p.rowwise_data for p in a], [p.rowwise_scale for p in a],
                        [w.rowwise_data for w in ws], [w.rowwise_scale for w in ws], dtype, outs=outs)


def _gemm_desc(qa, sa, qb, sb, dtype, out):
    """The C descriptor of one product, and its output tensor."""
    _out_code(dtype)
    qa2 = _as2d(qa, "qa", torch.uint8)
    qb2 = _as2d(qb, "qb", torch.uint8, device=qa.device)
    M, K = qa2.shape
    N = qb2.shape[0]
    if qb2.shape[1] != K:
        raise ValueError("gemm: planes must be qa [M, K], sa [M, K/32], qb [N, K], sb [N, K/32]")
    # scale planes may be views of padded allocations (rows a pitch apart) or
    # 3-D planes in the MFMA order
    sa2, pa = _scale_pitch(sa, (M, K // BLOCK), qa.device, "sa", allocate=False)
    sb2, pb = _scale_pitch(sb, (N, K // BLOCK), qa.device, "sb", allocate=False)
    # out may be a column slice of a wider matrix: rows stride(0) elements apart
    if out is None:
        o, po = torch.empty((M, N), dtype=dtype, device=qa.device), 0
    else:
        o = out
        if (tuple(o.shape) != (M, N) or o.dtype != dtype or o.device != qa.device
                or (N > 1 and o.stride(1) != 1) or (M > 1 and o.stride(0) < N)):
            raise ValueError("out must be a %s tensor of shape %s on %s with unit column stride and a "
                             "row stride >= %d" % (dtype, (M, N), qa.device, N))
        po = o.stride(0) if M > 1 and o.stride(0) != N else 0
    return _GemmDesc(_ptr(qa2), _ptr(sa2), _ptr(qb2), _ptr(sb2), M, N, K, pa, pb, _ptr(o), po), o

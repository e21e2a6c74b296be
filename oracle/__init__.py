"""CPU oracle for MXFP8 block quantization (test infrastructure only).

This package is the plain, slow definition the GPU library is checked
against.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the library itself never does and shares no
code with it.  The arithmetic lives in ``mxfp8_oracle.c`` (plain C, double
precision, scalar loops); this module only builds it and marshals numpy
arrays.

Arrays are numpy: bf16 tensors are passed as their ``uint16`` bit patterns,
e4m3 and e8m0 planes as ``uint8`` bytes.  Shapes follow the pages:

* rowwise scales ``[rows, cols/32]`` (Mojo DistributedAllGatherRMSNormQuantMXFP8
  page, "Args", outputs_scale);
* columnwise scales ``[rows/32, cols]`` (Megatron-Core quantized_dbuffer page,
  API, _block_atomic_to_flat: one columnwise scale row per 32-row block);
* both data planes ``[rows, cols]``, not transposed (quantized_dbuffer page,
  Functions, _rowwise_scale_layout / _columnwise_scale_layout).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxfp8_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmxfp8_oracle.so")
SOURCE = _SRC
BLOCK = 32


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the C oracle with gcc (no fast-math); returns the library path."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
             "-Wall", "-Wextra", "-o", tmp, src, "-lm"])
        os.replace(tmp, out)
    return out


def _values(x):
    """bf16 bit patterns (uint16) or float32 values, contiguous; the suffix of
    the C function that takes them."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, ""
    if x.dtype == np.float32:
        return x, "_f32"
    raise TypeError("inputs are bf16 bit patterns (uint16) or float32, got %s" % x.dtype)


def _bits16(x) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("bf16 inputs are passed as uint16 bit patterns, got %s" % x.dtype)
    return x


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


class Oracle:
    """The oracle's functions, bound to one compiled copy of mxfp8_oracle.c."""

    _SIGS = {
        "mxfp8_oracle_quantize_rowwise": "p i64 i64 p p",
        "mxfp8_oracle_quantize_colwise": "p i64 i64 p p",
        "mxfp8_oracle_quantize_rowwise_f32": "p i64 i64 p p",
        "mxfp8_oracle_quantize_colwise_f32": "p i64 i64 p p",
        "mxfp8_oracle_dequantize": "p p i64 i64 i32 p",
        "mxfp8_oracle_round_bf16": "p i64 p",
        "mxfp8_oracle_rmsnorm_f64": "p p f32 f32 i64 i64 p",
        "mxfp8_oracle_rmsnorm": "p p f32 f32 i64 i64 p",
        "mxfp8_oracle_rmsnorm_quantize": "p p f32 f32 i64 i64 p p p",
        "mxfp8_oracle_gemm": "p p p p i64 i64 i64 p p",
        "mxfp8_oracle_gemm_at": "p p p p i64 p p i64 p p",
        "mxfp8_oracle_set_threads": "i32",
        "mxfp8_oracle_max_threads": "",
    }
    _CT = {"p": ctypes.c_void_p, "i64": ctypes.c_int64, "i32": ctypes.c_int,
           "f32": ctypes.c_float}

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        for name, sig in self._SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = [self._CT[t] for t in sig.split()]
            fn.restype = ctypes.c_int if name == "mxfp8_oracle_max_threads" else None
        self.lib = lib
        self.path = lib_path

    def set_threads(self, n: int) -> None:
        self.lib.mxfp8_oracle_set_threads(int(n))

    def max_threads(self) -> int:
        return int(self.lib.mxfp8_oracle_max_threads())

    def quantize_rowwise(self, x):
        """Rowwise plane of a [rows, cols] tensor given as bf16 bit patterns
        (uint16) or float32: (q [rows, cols], s [rows, cols/32])."""
        x, sfx = _values(x)
        rows, cols = x.shape
        if cols % BLOCK:
            raise ValueError("cols must be a multiple of 32")
        q = np.empty((rows, cols), np.uint8)
        s = np.empty((rows, cols // BLOCK), np.uint8)
        getattr(self.lib, "mxfp8_oracle_quantize_rowwise" + sfx)(_ptr(x), rows, cols, _ptr(q), _ptr(s))
        return q, s

    def quantize_colwise(self, x):
        """Columnwise plane of a [rows, cols] tensor given as bf16 bit patterns
        (uint16) or float32: (q [rows, cols], s [rows/32, cols])."""
        x, sfx = _values(x)
        rows, cols = x.shape
        if rows % BLOCK:
            raise ValueError("rows must be a multiple of 32")
        q = np.empty((rows, cols), np.uint8)
        s = np.empty((rows // BLOCK, cols), np.uint8)
        getattr(self.lib, "mxfp8_oracle_quantize_colwise" + sfx)(_ptr(x), rows, cols, _ptr(q), _ptr(s))
        return q, s

    def quantize_colwise_t(self, x):
        """The columnwise plane stored transposed (the library's
        MXFP8_COLUMNWISE_T layout): q_t [cols, rows] with q_t[c, r] = q[r, c]
        and s_t [cols, rows/32] with s_t[c, b] = s[b, c], for (q, s) the
        columnwise plane above."""
        q, s = self.quantize_colwise(x)
        return np.ascontiguousarray(q.T), np.ascontiguousarray(s.T)

    def dequantize(self, q, s, axis: int):
        """Exact float64 values of a plane; axis 0 = rowwise scales, 1 = columnwise."""
        q = np.ascontiguousarray(q, np.uint8)
        s = np.ascontiguousarray(s, np.uint8)
        rows, cols = q.shape
        want = (rows, cols // BLOCK) if axis == 0 else (rows // BLOCK, cols)
        if s.shape != want:
            raise ValueError("scale shape %s, expected %s" % (s.shape, want))
        out = np.empty((rows, cols), np.float64)
        self.lib.mxfp8_oracle_dequantize(_ptr(q), _ptr(s), rows, cols, int(axis), _ptr(out))
        return out

    def gemm(self, qa, sa, qb, sb):
        """(C, abs_sum): C[m, n] = sum_k A[m, k] B[n, k] in float64 for rowwise
        planes A (qa [M, K], sa [M, K/32]) and B (qb [N, K], sb [N, K/32]);
        abs_sum[m, n] = sum_k |A[m, k] B[n, k]|."""
        qa, sa, qb, sb = (np.ascontiguousarray(t, np.uint8) for t in (qa, sa, qb, sb))
        M, K = qa.shape
        N = qb.shape[0]
        if qb.shape[1] != K or K % BLOCK or sa.shape != (M, K // BLOCK) or sb.shape != (N, K // BLOCK):
            raise ValueError("bad plane shapes")
        out = np.empty((M, N), np.float64)
        mag = np.empty((M, N), np.float64)
        self.lib.mxfp8_oracle_gemm(_ptr(qa), _ptr(sa), _ptr(qb), _ptr(sb), M, N, K, _ptr(out), _ptr(mag))
        return out, mag

    def gemm_at(self, qa, sa, qb, sb, ms, ns):
        """The same product at positions (ms[i], ns[i]) only."""
        qa, sa, qb, sb = (np.ascontiguousarray(t, np.uint8) for t in (qa, sa, qb, sb))
        M, K = qa.shape
        N = qb.shape[0]
        ms = np.ascontiguousarray(ms, np.int64)
        ns = np.ascontiguousarray(ns, np.int64)
        if qb.shape[1] != K or ms.shape != ns.shape or (ms >= M).any() or (ns >= N).any():
            raise ValueError("bad plane shapes or positions")
        out = np.empty(ms.shape, np.float64)
        mag = np.empty(ms.shape, np.float64)
        self.lib.mxfp8_oracle_gemm_at(_ptr(qa), _ptr(sa), _ptr(qb), _ptr(sb), K, _ptr(ms), _ptr(ns),
                                      ms.size, _ptr(out), _ptr(mag))
        return out, mag

    def round_bf16(self, v):
        """bf16 bit patterns of float64 values, round to nearest even."""
        v = np.ascontiguousarray(v, np.float64)
        out = np.empty(v.shape, np.uint16)
        self.lib.mxfp8_oracle_round_bf16(_ptr(v), v.size, _ptr(out))
        return out

    def _norm_args(self, x_bits, gamma_bits):
        x = _bits16(x_bits)
        g = _bits16(gamma_bits)
        rows, cols = x.shape
        if g.shape != (cols,):
            raise ValueError("gamma must have shape [cols]")
        return x, g, rows, cols

    def rmsnorm_f64(self, x_bits, gamma_bits, weight_offset: float, eps: float):
        """RMSNorm rows in float64, before rounding to bf16."""
        x, g, rows, cols = self._norm_args(x_bits, gamma_bits)
        y = np.empty((rows, cols), np.float64)
        self.lib.mxfp8_oracle_rmsnorm_f64(_ptr(x), _ptr(g), float(weight_offset),
                                          float(eps), rows, cols, _ptr(y))
        return y

    def rmsnorm(self, x_bits, gamma_bits, weight_offset: float, eps: float):
        """RMSNorm rows rounded once to bf16 (uint16 bit patterns)."""
        x, g, rows, cols = self._norm_args(x_bits, gamma_bits)
        out = np.empty((rows, cols), np.uint16)
        self.lib.mxfp8_oracle_rmsnorm(_ptr(x), _ptr(g), float(weight_offset), float(eps),
                                      rows, cols, _ptr(out))
        return out

    def rmsnorm_quantize(self, x_bits, gamma_bits, weight_offset: float, eps: float):
        """(normed bf16 bits, q [rows, cols], s [rows, cols/32]) of the fused op."""
        x, g, rows, cols = self._norm_args(x_bits, gamma_bits)
        if cols % BLOCK:
            raise ValueError("cols must be a multiple of 32")
        normed = np.empty((rows, cols), np.uint16)
        q = np.empty((rows, cols), np.uint8)
        s = np.empty((rows, cols // BLOCK), np.uint8)
        self.lib.mxfp8_oracle_rmsnorm_quantize(_ptr(x), _ptr(g), float(weight_offset),
                                               float(eps), rows, cols, _ptr(normed),
                                               _ptr(q), _ptr(s))
        return normed, q, s


_default = None


def default() -> Oracle:
    """The oracle built from this directory's source (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _default = Oracle(_LIB_PATH)
    return _default


def __getattr__(name):
    # Module-level access (oracle.quantize_rowwise, ...) goes to the default build.
    if name in ("set_threads", "max_threads", "quantize_rowwise", "quantize_colwise",
                "dequantize", "round_bf16", "rmsnorm_f64", "rmsnorm", "rmsnorm_quantize",
                "gemm", "gemm_at"):
        return getattr(default(), name)
    raise AttributeError(name)

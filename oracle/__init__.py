"""CPU oracle for int8 weight-only quantization, the W8A16 matmul and the
W8A8 (int8 x int8) matmul.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The
product library (``int8_weight_quantized_amd``) never imports, links or
calls it, and the two share no code: this package wraps the plain C file
``qw_oracle.c`` (built with gcc, no FMA contraction, no fast-math) through
ctypes and converts numpy arrays to and from its pointer arguments.

What each function computes is stated in ``qw_oracle.c`` together with the
passages of the pages it follows; this wrapper does no arithmetic of the
method.  Parity status: every exported function is pinned by the
``-m "not gpu"`` tests in ``tests/test_oracle_*.py`` (library special
cases, brute force with exact rationals, invariants, closed forms and the
pages' worked example); none is "parity unpinned".
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "qw_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")
# QW_ORACLE_LIBRARY names another build of the oracle (the sanitizer test
# loads an AddressSanitizer / UBSan build this way); it is used as is.
_OVERRIDE = os.environ.get("QW_ORACLE_LIBRARY")

# -ffp-contract=off: no fused multiply-add may merge two IEEE operations.
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
          "-fno-strict-aliasing", "-fopenmp", "-shared", "-fPIC", "-Wall"]

_lock = threading.Lock()
_lib = None


def build(source: str = SOURCE, output: str = LIBRARY, extra_flags=()) -> str:
    """Compile the oracle C file into a shared library with gcc."""
    tmp = output + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *extra_flags, source, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, output)
    return output


def _needs_build(output: str = LIBRARY) -> bool:
    if not os.path.exists(output):
        return True
    return os.path.getmtime(output) < os.path.getmtime(SOURCE)


def _declare(lib):
    i64, u16p, f32p, f64p, i8p, i64p = (
        ctypes.c_int64, ctypes.POINTER(ctypes.c_uint16),
        ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double),
        ctypes.POINTER(ctypes.c_int8), ctypes.POINTER(ctypes.c_int64))
    lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_f16.restype = ctypes.c_uint16
    lib.oracle_f64_to_f16.argtypes = [ctypes.c_double]
    lib.oracle_f64_to_f16.restype = ctypes.c_uint16
    lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_f16_array.argtypes = [f32p, u16p, i64]
    lib.oracle_f64_to_f16_array.argtypes = [f64p, u16p, i64]
    lib.oracle_f16_to_f32_array.argtypes = [u16p, f32p, i64]
    lib.oracle_row_percentile.argtypes = [f32p, i64, ctypes.c_double, f32p]
    lib.oracle_row_percentile.restype = ctypes.c_double
    lib.oracle_quantize.argtypes = [f32p, i64, i64, ctypes.c_double, i8p, u16p, f32p]
    lib.oracle_quantize.restype = ctypes.c_int
    lib.oracle_gemm.argtypes = [u16p, i8p, u16p, i64, i64, i64, f64p]
    lib.oracle_gemm_sampled.argtypes = [u16p, i8p, u16p, i64, i64p, i64p, i64, f64p]
    lib.oracle_quantize_asym.argtypes = [f32p, i64, i64, i8p, u16p, i8p]
    lib.oracle_quantize_asym.restype = ctypes.c_int
    lib.oracle_gemm_asym.argtypes = [u16p, i8p, u16p, i8p, i64, i64, i64, f64p]
    lib.oracle_gemm_asym_sampled.argtypes = [u16p, i8p, u16p, i8p, i64, i64p, i64p, i64, f64p]
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.oracle_quantize_outliers.argtypes = [f32p, i64, i64, ctypes.c_double, i8p, u16p, i32p, f32p, i64]
    lib.oracle_quantize_outliers.restype = ctypes.c_int
    lib.oracle_outlier_capacity.argtypes = [i64, ctypes.c_double]
    lib.oracle_outlier_capacity.restype = ctypes.c_int64
    lib.oracle_gemm_outliers.argtypes = [u16p, i8p, u16p, i32p, f32p, i64, i64, i64, i64, f64p]
    lib.oracle_gemm_outliers_sampled.argtypes = [u16p, i8p, u16p, i32p, f32p, i64, i64, i64p, i64p, i64, f64p]
    lib.oracle_quantize_fixed.argtypes = [f32p, i64, i64, f32p, i8p, u16p]
    lib.oracle_quantize_fixed.restype = ctypes.c_int
    lib.oracle_w8a8_gemm.argtypes = [i8p, u16p, i8p, u16p, i64, i64, i64, f64p]
    lib.oracle_w8a8_gemm_sampled.argtypes = [i8p, u16p, i8p, u16p, i64, i64p, i64p, i64, f64p]
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def load_library(path: str):
    """Load an oracle build (the default one, or a variant a test compiled)."""
    return _declare(ctypes.CDLL(path))


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if _OVERRIDE:
                _lib = load_library(_OVERRIDE)
            else:
                if _needs_build():
                    build()
                _lib = load_library(LIBRARY)
    return _lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


class Oracle:
    """numpy-facing wrapper around one oracle build."""

    def __init__(self, cdll=None):
        self._l = cdll if cdll is not None else lib()

    # --- binary16 conversions --------------------------------------------
    def f32_to_f16_bits(self, x) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint16)
        self._l.oracle_f32_to_f16_array(_ptr(x, ctypes.c_float), _ptr(out, ctypes.c_uint16), x.size)
        return out

    def f64_to_f16_bits(self, x) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(x.shape, dtype=np.uint16)
        self._l.oracle_f64_to_f16_array(_ptr(x, ctypes.c_double), _ptr(out, ctypes.c_uint16), x.size)
        return out

    def f16_bits_to_f32(self, h) -> np.ndarray:
        h = np.ascontiguousarray(h, dtype=np.uint16)
        out = np.empty(h.shape, dtype=np.float32)
        self._l.oracle_f16_to_f32_array(_ptr(h, ctypes.c_uint16), _ptr(out, ctypes.c_float), h.size)
        return out

    # --- threshold, quantizer, matmul ------------------------------------
    def row_percentile(self, row, pct: float) -> float:
        """Binary64 type-7 percentile of |row| (the unrounded clip bound)."""
        row = np.ascontiguousarray(row, dtype=np.float32).ravel()
        scratch = np.empty_like(row)
        return self._l.oracle_row_percentile(_ptr(row, ctypes.c_float), row.size, float(pct),
                                             _ptr(scratch, ctypes.c_float))

    def quantize(self, w, pct: float = 100.0):
        """Return (q int8 [n,k], scale fp16 bits uint16 [n], threshold f32 [n])."""
        w = np.ascontiguousarray(w, dtype=np.float32)
        if w.ndim != 2:
            raise ValueError("w must be 2-D [n, k]")
        n, k = w.shape
        q = np.empty((n, k), dtype=np.int8)
        s = np.empty((n,), dtype=np.uint16)
        t = np.empty((n,), dtype=np.float32)
        rc = self._l.oracle_quantize(_ptr(w, ctypes.c_float), n, k, float(pct),
                                     _ptr(q, ctypes.c_int8), _ptr(s, ctypes.c_uint16),
                                     _ptr(t, ctypes.c_float))
        if rc != 0:
            raise ValueError("oracle_quantize rejected its arguments (rc=%d)" % rc)
        return q, s, t

    def quantize_fixed(self, w, bounds):
        """Per-row quantization with given bounds (fixed-range clip):
        returns (q int8 [n,k], scale bits uint16 [n])."""
        w = np.ascontiguousarray(w, dtype=np.float32)
        b = np.ascontiguousarray(bounds, dtype=np.float32)
        n, k = w.shape
        if b.shape != (n,):
            raise ValueError("bounds must be [n]")
        q = np.empty((n, k), dtype=np.int8)
        s = np.empty((n,), dtype=np.uint16)
        rc = self._l.oracle_quantize_fixed(_ptr(w, ctypes.c_float), n, k, _ptr(b, ctypes.c_float),
                                           _ptr(q, ctypes.c_int8), _ptr(s, ctypes.c_uint16))
        if rc != 0:
            raise ValueError("oracle_quantize_fixed rejected its arguments (rc=%d)" % rc)
        return q, s

    def outlier_capacity(self, k: int, pct: float) -> int:
        return int(self._l.oracle_outlier_capacity(k, float(pct)))

    def quantize_outliers(self, w, pct: float, cap: int = None):
        """Outlier-aware quantization: returns (q int8 [n,k], scale bits uint16
        [n], outlier columns int32 [n,cap] (-1 unused), outlier values float32
        [n,cap])."""
        w = np.ascontiguousarray(w, dtype=np.float32)
        n, k = w.shape
        if cap is None:
            cap = self.outlier_capacity(k, pct)
        q = np.empty((n, k), dtype=np.int8)
        s = np.empty((n,), dtype=np.uint16)
        idx = np.empty((n, cap), dtype=np.int32)
        val = np.empty((n, cap), dtype=np.float32)
        rc = self._l.oracle_quantize_outliers(_ptr(w, ctypes.c_float), n, k, float(pct), _ptr(q, ctypes.c_int8),
                                              _ptr(s, ctypes.c_uint16), _ptr(idx, ctypes.c_int32),
                                              _ptr(val, ctypes.c_float), cap)
        if rc != 0:
            raise ValueError("oracle_quantize_outliers rejected its arguments (rc=%d)" % rc)
        return q, s, idx, val

    def gemm_outliers(self, x_f16, q, s_bits, idx, val) -> np.ndarray:
        x = np.ascontiguousarray(np.asarray(x_f16, dtype=np.float16)).view(np.uint16)
        q = np.ascontiguousarray(q, dtype=np.int8)
        s = np.ascontiguousarray(s_bits, dtype=np.uint16)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        val = np.ascontiguousarray(val, dtype=np.float32)
        m, k = x.shape
        n = q.shape[0]
        cap = idx.shape[1] if idx.ndim == 2 else 0
        if q.shape != (n, k) or s.shape != (n,) or idx.shape != (n, cap) or val.shape != (n, cap):
            raise ValueError("shape mismatch")
        if cap and (idx.max() >= k or idx.min() < -1):
            raise IndexError("outlier column out of range")
        ref = np.empty((m, n), dtype=np.float64)
        self._l.oracle_gemm_outliers(_ptr(x, ctypes.c_uint16), _ptr(q, ctypes.c_int8), _ptr(s, ctypes.c_uint16),
                                     _ptr(idx, ctypes.c_int32), _ptr(val, ctypes.c_float), cap, m, n, k,
                                     _ptr(ref, ctypes.c_double))
        return ref

    def gemm_outliers_sampled(self, x_f16, q, s_bits, idx, val, mi, ni) -> np.ndarray:
        x = np.ascontiguousarray(np.asarray(x_f16, dtype=np.float16)).view(np.uint16)
        q = np.ascontiguousarray(q, dtype=np.int8)
        s = np.ascontiguousarray(s_bits, dtype=np.uint16)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        val = np.ascontiguousarray(val, dtype=np.float32)
        mi = np.ascontiguousarray(mi, dtype=np.int64)
        ni = np.ascontiguousarray(ni, dtype=np.int64)
        k = x.shape[1]
        cap = idx.shape[1]
        if q.shape[1] != k or mi.shape != ni.shape or idx.shape != (q.shape[0], cap) or val.shape != idx.shape:
            raise ValueError("shape mismatch")
        if mi.size and (mi.min() < 0 or mi.max() >= x.shape[0] or ni.min() < 0 or ni.max() >= q.shape[0]):
            raise IndexError("sample index out of range")
        if cap and (idx.max() >= k or idx.min() < -1):
            raise IndexError("outlier column out of range")
        out = np.empty(mi.shape, dtype=np.float64)
        self._l.oracle_gemm_outliers_sampled(_ptr(x, ctypes.c_uint16), _ptr(q, ctypes.c_int8),
                                             _ptr(s, ctypes.c_uint16), _ptr(idx, ctypes.c_int32),
                                             _ptr(val, ctypes.c_float), cap, k, _ptr(mi, ctypes.c_int64),
                                             _ptr(ni, ctypes.c_int64), mi.size, _ptr(out, ctypes.c_double))
        return out

    def quantize_asym(self, w):
        """Asymmetric per-row quantization: returns (q int8 [n,k], scale bits
        uint16 [n], zero points int8 [n])."""
        w = np.ascontiguousarray(w, dtype=np.float32)
        n, k = w.shape
        q = np.empty((n, k), dtype=np.int8)
        s = np.empty((n,), dtype=np.uint16)
        z = np.empty((n,), dtype=np.int8)
        rc = self._l.oracle_quantize_asym(_ptr(w, ctypes.c_float), n, k, _ptr(q, ctypes.c_int8),
                                          _ptr(s, ctypes.c_uint16), _ptr(z, ctypes.c_int8))
        if rc != 0:
            raise ValueError("oracle_quantize_asym rejected its arguments (rc=%d)" % rc)
        return q, s, z

    def gemm_asym(self, x_f16, q, s_bits, zeros) -> np.ndarray:
        """Binary64 reference ref[m, n] = sum_k x[m,k] * (q[n,k] - z[n]) * S[n]."""
        x = np.ascontiguousarray(np.asarray(x_f16, dtype=np.float16)).view(np.uint16)
        q = np.ascontiguousarray(q, dtype=np.int8)
        s = np.ascontiguousarray(s_bits, dtype=np.uint16)
        z = np.ascontiguousarray(zeros, dtype=np.int8)
        m, k = x.shape
        n = q.shape[0]
        if q.shape != (n, k) or s.shape != (n,) or z.shape != (n,):
            raise ValueError("shape mismatch")
        ref = np.empty((m, n), dtype=np.float64)
        self._l.oracle_gemm_asym(_ptr(x, ctypes.c_uint16), _ptr(q, ctypes.c_int8), _ptr(s, ctypes.c_uint16),
                                 _ptr(z, ctypes.c_int8), m, n, k, _ptr(ref, ctypes.c_double))
        return ref

    def gemm_asym_sampled(self, x_f16, q, s_bits, zeros, mi, ni) -> np.ndarray:
        x = np.ascontiguousarray(np.asarray(x_f16, dtype=np.float16)).view(np.uint16)
        q = np.ascontiguousarray(q, dtype=np.int8)
        s = np.ascontiguousarray(s_bits, dtype=np.uint16)
        z = np.ascontiguousarray(zeros, dtype=np.int8)
        mi = np.ascontiguousarray(mi, dtype=np.int64)
        ni = np.ascontiguousarray(ni, dtype=np.int64)
        k = x.shape[1]
        if q.shape[1] != k or mi.shape != ni.shape or z.shape != (q.shape[0],):
            raise ValueError("shape mismatch")
        if mi.size and (mi.min() < 0 or mi.max() >= x.shape[0] or ni.min() < 0 or ni.max() >= q.shape[0]):
            raise IndexError("sample index out of range")
        out = np.empty(mi.shape, dtype=np.float64)
        self._l.oracle_gemm_asym_sampled(_ptr(x, ctypes.c_uint16), _ptr(q, ctypes.c_int8),
                                         _ptr(s, ctypes.c_uint16), _ptr(z, ctypes.c_int8), k,
                                         _ptr(mi, ctypes.c_int64), _ptr(ni, ctypes.c_int64), mi.size,
                                         _ptr(out, ctypes.c_double))
        return out

    def gemm(self, x_f16, q, s_bits) -> np.ndarray:
        """Binary64 reference ref[m, n] = sum_k x[m,k] * q[n,k] * S[n]."""
        x = np.ascontiguousarray(np.asarray(x_f16, dtype=np.float16)).view(np.uint16)
        q = np.ascontiguousarray(q, dtype=np.int8)
        s = np.ascontiguousarray(s_bits, dtype=np.uint16)
        m, k = x.shape
        n = q.shape[0]
        if q.shape != (n, k) or s.shape != (n,):
            raise ValueError("shape mismatch")
        ref = np.empty((m, n), dtype=np.float64)
        self._l.oracle_gemm(_ptr(x, ctypes.c_uint16), _ptr(q, ctypes.c_int8),
                            _ptr(s, ctypes.c_uint16), m, n, k, _ptr(ref, ctypes.c_double))
        return ref

    def gemm_sampled(self, x_f16, q, s_bits, mi, ni) -> np.ndarray:
        """ref[mi[c], ni[c]] for each c, computed one output at a time."""
        x = np.ascontiguousarray(np.asarray(x_f16, dtype=np.float16)).view(np.uint16)
        q = np.ascontiguousarray(q, dtype=np.int8)
        s = np.ascontiguousarray(s_bits, dtype=np.uint16)
        mi = np.ascontiguousarray(mi, dtype=np.int64)
        ni = np.ascontiguousarray(ni, dtype=np.int64)
        k = x.shape[1]
        if q.shape[1] != k or mi.shape != ni.shape:
            raise ValueError("shape mismatch")
        if mi.size and (mi.min() < 0 or mi.max() >= x.shape[0] or ni.min() < 0 or ni.max() >= q.shape[0]):
            raise IndexError("sample index out of range")
        out = np.empty(mi.shape, dtype=np.float64)
        self._l.oracle_gemm_sampled(_ptr(x, ctypes.c_uint16), _ptr(q, ctypes.c_int8),
                                    _ptr(s, ctypes.c_uint16), k, _ptr(mi, ctypes.c_int64),
                                    _ptr(ni, ctypes.c_int64), mi.size, _ptr(out, ctypes.c_double))
        return out

    def w8a8_gemm(self, qx, sx_bits, q, s_bits) -> np.ndarray:
        """Binary64 reference ref[m, n] = (sum_k qx[m,k] q[n,k]) * Sx[m] * S[n]."""
        qx = np.ascontiguousarray(qx, dtype=np.int8)
        sx = np.ascontiguousarray(sx_bits, dtype=np.uint16)
        q = np.ascontiguousarray(q, dtype=np.int8)
        s = np.ascontiguousarray(s_bits, dtype=np.uint16)
        m, k = qx.shape
        n = q.shape[0]
        if q.shape != (n, k) or s.shape != (n,) or sx.shape != (m,):
            raise ValueError("shape mismatch")
        ref = np.empty((m, n), dtype=np.float64)
        self._l.oracle_w8a8_gemm(_ptr(qx, ctypes.c_int8), _ptr(sx, ctypes.c_uint16),
                                 _ptr(q, ctypes.c_int8), _ptr(s, ctypes.c_uint16), m, n, k,
                                 _ptr(ref, ctypes.c_double))
        return ref

    def w8a8_gemm_sampled(self, qx, sx_bits, q, s_bits, mi, ni) -> np.ndarray:
        """W8A8 ref[mi[c], ni[c]] for each c, computed one output at a time."""
        qx = np.ascontiguousarray(qx, dtype=np.int8)
        sx = np.ascontiguousarray(sx_bits, dtype=np.uint16)
        q = np.ascontiguousarray(q, dtype=np.int8)
        s = np.ascontiguousarray(s_bits, dtype=np.uint16)
        mi = np.ascontiguousarray(mi, dtype=np.int64)
        ni = np.ascontiguousarray(ni, dtype=np.int64)
        k = qx.shape[1]
        if q.shape[1] != k or mi.shape != ni.shape or sx.shape != (qx.shape[0],) or s.shape != (q.shape[0],):
            raise ValueError("shape mismatch")
        if mi.size and (mi.min() < 0 or mi.max() >= qx.shape[0] or ni.min() < 0 or ni.max() >= q.shape[0]):
            raise IndexError("sample index out of range")
        out = np.empty(mi.shape, dtype=np.float64)
        self._l.oracle_w8a8_gemm_sampled(_ptr(qx, ctypes.c_int8), _ptr(sx, ctypes.c_uint16),
                                         _ptr(q, ctypes.c_int8), _ptr(s, ctypes.c_uint16), k,
                                         _ptr(mi, ctypes.c_int64), _ptr(ni, ctypes.c_int64), mi.size,
                                         _ptr(out, ctypes.c_double))
        return out

    def num_threads(self) -> int:
        return int(self._l.oracle_num_threads())


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def quantize(w, pct: float = 100.0):
    return default().quantize(w, pct)


def quantize_fixed(w, bounds):
    return default().quantize_fixed(w, bounds)


def outlier_capacity(k, pct):
    return default().outlier_capacity(k, pct)


def quantize_outliers(w, pct, cap=None):
    return default().quantize_outliers(w, pct, cap)


def gemm_outliers(x_f16, q, s_bits, idx, val):
    return default().gemm_outliers(x_f16, q, s_bits, idx, val)


def gemm_outliers_sampled(x_f16, q, s_bits, idx, val, mi, ni):
    return default().gemm_outliers_sampled(x_f16, q, s_bits, idx, val, mi, ni)


def quantize_asym(w):
    return default().quantize_asym(w)


def gemm_asym(x_f16, q, s_bits, zeros):
    return default().gemm_asym(x_f16, q, s_bits, zeros)


def gemm_asym_sampled(x_f16, q, s_bits, zeros, mi, ni):
    return default().gemm_asym_sampled(x_f16, q, s_bits, zeros, mi, ni)


def gemm(x_f16, q, s_bits):
    return default().gemm(x_f16, q, s_bits)


def gemm_sampled(x_f16, q, s_bits, mi, ni):
    return default().gemm_sampled(x_f16, q, s_bits, mi, ni)


def w8a8_gemm(qx, sx_bits, q, s_bits):
    return default().w8a8_gemm(qx, sx_bits, q, s_bits)


def w8a8_gemm_sampled(qx, sx_bits, q, s_bits, mi, ni):
    return default().w8a8_gemm_sampled(qx, sx_bits, q, s_bits, mi, ni)


def f64_to_f16_bits(x):
    return default().f64_to_f16_bits(x)


def f16_bits_to_f32(h):
    return default().f16_bits_to_f32(h)

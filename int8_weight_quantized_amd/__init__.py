"""int8 weight-only (W8A16) Linear layers for AMD Instinct MI355X (gfx950).

A thin Python binding over the C ABI of ``libqw.so`` (declared in
``include/qw.h``).  This module only marshals arguments: it checks tensor
dtypes, shapes and devices, allocates outputs with torch, and passes raw
device pointers plus the current HIP stream to the library.  Every step of
the computation runs in the library's HIP kernels; there is no CPU or
PyTorch fallback, and importing this package fails loudly when the library
has not been built (``python -m int8_weight_quantized_amd.build``): the
first call, or ``library()``, raises ImportError.

    q, s = quantize_weights(w)              # w: cuda fp32 [N, K]
    y = w8a16_gemm(x, q, s)                 # x: cuda fp16 [M, K] -> fp16 [M, N]

Names follow the pages: symmetric per-channel int8 weight quantization with
an optional percentage clip (LightSeq slide deck, "量化流程" and
"量化：裁剪+对称") and the W8A16 MatMul whose right operand is the int8
weight ("探索ChatGLM2在算能BM1684X上INT8量化部署", sections 2-4).
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# QW_LIBRARY names another build of the same library (the CPU tests load a
# host-sanitizer build this way).
LIBRARY_PATH = os.environ.get("QW_LIBRARY") or os.path.join(HERE, "libqw.so")

QW_SUCCESS = 0
QW_ERROR_INVALID_VALUE = 1
QW_ERROR_MISALIGNED = 2
QW_ERROR_UNSUPPORTED = 3
QW_ERROR_LAUNCH = 4

PATHS = {"auto": 0, "gemv": 1, "mfma": 2, "skinny": 3}
QUANTIZE_MAX_K = 65536
MFMA_MAX_K = 8388608     # longest reduction of the LDS-tiled MFMA kernel
PINGPONG_MAX_K = 4194304  # longest reduction of the 256 x 256 ping-pong tile
MFMA_TILES = ((256, 256), (256, 128), (256, 64), (128, 128), (128, 64))  # (BN, BM)
W8A8_TILES = ((256, 256), (256, 128), (256, 64), (128, 64))
W8A8_MAX_K = 131072


class QwError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (where, status_string(status), status))


_lib_handle = None


def _load():
    """Load libqw.so once; raises ImportError when it has not been built."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(LIBRARY_PATH):
        raise ImportError(
            "libqw.so is not built (expected at %s); run `python -m int8_weight_quantized_amd.build`"
            % LIBRARY_PATH)
    # One HIP runtime per process: torch ships its own libamdhip64.so.7 and
    # loads it under a different file name, so if libqw.so were loaded
    # first the process would map two runtimes and torch's would find no
    # GPU.  Importing torch first makes the loader resolve libqw.so's
    # dependency (by soname) to the runtime torch already loaded, which is
    # also what makes torch's stream handles valid here.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIBRARY_PATH)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.qw_quantize_weights.argtypes = [vp, i64, i64, ctypes.c_double, vp, vp, vp]
    lib.qw_quantize_weights.restype = ctypes.c_int
    lib.qw_quantize_weights_f16.argtypes = [vp, i64, i64, ctypes.c_double, vp, vp, vp]
    lib.qw_quantize_weights_f16.restype = ctypes.c_int
    lib.qw_quantize_weights_fixed_range.argtypes = [vp, i64, i64, vp, vp, vp, vp]
    lib.qw_quantize_weights_fixed_range.restype = ctypes.c_int
    lib.qw_w8a16_gemm_tune.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
    lib.qw_w8a16_gemm_tune.restype = ctypes.c_int
    lib.qw_w8a16_gemm_tuned_choice.argtypes = [i64, i64, i64]
    lib.qw_w8a16_gemm_tuned_choice.restype = ctypes.c_int
    lib.qw_w8a16_gemm_tune_reset.argtypes = []
    lib.qw_w8a16_gemm_tune_reset.restype = None
    lib.qw_outlier_capacity.argtypes = [i64, ctypes.c_double]
    lib.qw_outlier_capacity.restype = ctypes.c_int64
    lib.qw_quantize_weights_outliers.argtypes = [vp, i64, i64, ctypes.c_double, vp, vp, vp, vp, i64, vp]
    lib.qw_quantize_weights_outliers.restype = ctypes.c_int
    lib.qw_w8a16_gemm_outliers.argtypes = [vp, vp, vp, vp, vp, i64, vp, i64, i64, i64, vp]
    lib.qw_w8a16_gemm_outliers.restype = ctypes.c_int
    lib.qw_w8a16_gemm_outliers_path.argtypes = [vp, vp, vp, vp, vp, i64, vp, i64, i64, i64, ctypes.c_int, vp]
    lib.qw_w8a16_gemm_outliers_path.restype = ctypes.c_int
    lib.qw_w8a16_gemm_tile.argtypes = [vp, vp, vp, vp, vp, vp, i64, vp, i64, i64, i64, ctypes.c_int, vp]
    lib.qw_w8a16_gemm_tile.restype = ctypes.c_int
    lib.qw_w8a8_gemm_tile.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, vp]
    lib.qw_w8a8_gemm_tile.restype = ctypes.c_int
    lib.qw_quantize_weights_asym.argtypes = [vp, i64, i64, vp, vp, vp, vp]
    lib.qw_quantize_weights_asym.restype = ctypes.c_int
    lib.qw_w8a16_gemm_asym.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp]
    lib.qw_w8a16_gemm_asym.restype = ctypes.c_int
    lib.qw_w8a16_gemm_asym_path.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, vp]
    lib.qw_w8a16_gemm_asym_path.restype = ctypes.c_int
    lib.qw_w8a8_gemm.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp]
    lib.qw_w8a8_gemm_path.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, vp]
    lib.qw_w8a8_gemm_path.restype = ctypes.c_int
    lib.qw_w8a8_gemm.restype = ctypes.c_int
    lib.qw_w8a8_gemm_mfma_tile.argtypes = [i64, i64, i64]
    lib.qw_w8a8_gemm_auto_path.argtypes = [i64, i64, i64]
    lib.qw_w8a8_gemm_auto_path.restype = ctypes.c_int
    lib.qw_w8a8_gemm_tune.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp]
    lib.qw_w8a8_gemm_tune.restype = ctypes.c_int
    lib.qw_w8a8_gemm_tuned_choice.argtypes = [i64, i64, i64]
    lib.qw_w8a8_gemm_tuned_choice.restype = ctypes.c_int
    lib.qw_w8a8_gemm_mfma_tile.restype = ctypes.c_int
    lib.qw_w8a16_gemm.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp]
    lib.qw_w8a16_gemm.restype = ctypes.c_int
    lib.qw_w8a16_gemm_path.argtypes = [vp, vp, vp, vp, i64, i64, i64, ctypes.c_int, vp]
    lib.qw_w8a16_gemm_path.restype = ctypes.c_int
    lib.qw_status_string.argtypes = [ctypes.c_int]
    lib.qw_status_string.restype = ctypes.c_char_p
    lib.qw_w8a16_gemm_auto_path.argtypes = [i64, i64, i64]
    lib.qw_w8a16_gemm_auto_path.restype = ctypes.c_int
    lib.qw_w8a16_gemm_mfma_tile.argtypes = [i64, i64, i64]
    lib.qw_w8a16_gemm_mfma_tile.restype = ctypes.c_int
    lib.qw_probe_stream_read.argtypes = [vp, i64, ctypes.c_uint32, vp, vp]
    lib.qw_probe_stream_read.restype = ctypes.c_int
    lib.qw_probe_shader_clock.argtypes = [vp, vp]
    lib.qw_probe_shader_clock.restype = ctypes.c_int
    lib.qw_version.argtypes = []
    lib.qw_version.restype = ctypes.c_int
    _lib_handle = lib
    return lib


def library():
    """The loaded ctypes handle of libqw.so (loads it on first use)."""
    return _load()


def status_string(status: int) -> str:
    return library().qw_status_string(int(status)).decode()


def version() -> int:
    return int(library().qw_version())


PATH_NAMES = {0: "auto", 1: "gemv", 2: "mfma", 3: "skinny"}


def auto_path(m: int, n: int, k: int) -> str:
    """Name of the kernel qw_w8a16_gemm runs for this shape."""
    p = int(library().qw_w8a16_gemm_auto_path(m, n, k))
    if p < 0:
        raise ValueError("unsupported GEMM shape m=%d n=%d k=%d" % (m, n, k))
    return PATH_NAMES[p]


def mfma_tile(m: int, n: int, k: int):
    """(BN, BM) output tile the MFMA kernel uses for this shape on the current
    device (needs a GPU)."""
    t = int(library().qw_w8a16_gemm_mfma_tile(m, n, k))
    if t < 0:
        raise ValueError("no MFMA tile for m=%d n=%d k=%d (bad shape or no device)" % (m, n, k))
    return t // 1000, t % 1000


def w8a8_auto_path(m: int, n: int, k: int) -> str:
    """Name of the kernel qw_w8a8_gemm runs for this shape."""
    p = int(library().qw_w8a8_gemm_auto_path(m, n, k))
    if p < 0:
        raise ValueError("unsupported W8A8 GEMM shape m=%d n=%d k=%d" % (m, n, k))
    return PATH_NAMES[p]


def w8a8_tile(m: int, n: int, k: int):
    """(BN, BM) output tile the W8A8 kernel uses for this shape on the
    current device (needs a GPU)."""
    t = int(library().qw_w8a8_gemm_mfma_tile(m, n, k))
    if t < 0:
        raise ValueError("no W8A8 tile for m=%d n=%d k=%d (bad shape or no device)" % (m, n, k))
    return t // 1000, t % 1000


# ---------------------------------------------------------------------------
# raw C-ABI calls (device pointers as ints); used by tests and the benchmark
# ---------------------------------------------------------------------------

def quantize_weights_raw(w_ptr: int, n: int, k: int, clip_percentile: float,
                         q_ptr: int, s_ptr: int, stream: int = 0) -> int:
    return int(library().qw_quantize_weights(w_ptr, n, k, float(clip_percentile), q_ptr, s_ptr, stream))


def quantize_weights_f16_raw(w_ptr: int, n: int, k: int, clip_percentile: float,
                             q_ptr: int, s_ptr: int, stream: int = 0) -> int:
    return int(library().qw_quantize_weights_f16(w_ptr, n, k, float(clip_percentile), q_ptr, s_ptr, stream))


def quantize_weights_fixed_range_raw(w_ptr: int, n: int, k: int, bounds_ptr: int, q_ptr: int, s_ptr: int,
                                     stream: int = 0) -> int:
    return int(library().qw_quantize_weights_fixed_range(w_ptr, n, k, bounds_ptr, q_ptr, s_ptr, stream))


def w8a16_gemm_tune_raw(x_ptr: int, q_ptr: int, s_ptr: int, y_ptr: int, m: int, n: int, k: int,
                        stream: int = 0) -> int:
    return int(library().qw_w8a16_gemm_tune(x_ptr, q_ptr, s_ptr, y_ptr, m, n, k, stream))


def _decode_choice(c: int):
    if c < 0:
        return None
    path, tile = divmod(c, 1000000)
    name = {v: k2 for k2, v in PATHS.items()}[path]
    return name, ((tile // 1000, tile % 1000) if tile else None)


def tuned_choice(m: int, n: int, k: int):
    """The W8A16 tuning record for the bucket of (m, n, k) on the current
    device: (path name, (BN, BM) or None), or None when the shape has none."""
    return _decode_choice(int(library().qw_w8a16_gemm_tuned_choice(m, n, k)))


def w8a8_tuned_choice(m: int, n: int, k: int):
    """The W8A8 tuning record for the bucket of (m, n, k), as tuned_choice."""
    return _decode_choice(int(library().qw_w8a8_gemm_tuned_choice(m, n, k)))


def tune_reset() -> None:
    """Forget every tuning record (W8A16 and W8A8)."""
    library().qw_w8a16_gemm_tune_reset()


def w8a8_gemm_tune_raw(qx_ptr: int, sx_ptr: int, q_ptr: int, s_ptr: int, y_ptr: int, m: int, n: int, k: int,
                       stream: int = 0) -> int:
    return int(library().qw_w8a8_gemm_tune(qx_ptr, sx_ptr, q_ptr, s_ptr, y_ptr, m, n, k, stream))


def outlier_capacity(k: int, clip_percentile: float) -> int:
    """Side-list slots per row that always hold the outliers (host only)."""
    c = int(library().qw_outlier_capacity(k, float(clip_percentile)))
    if c < 0:
        raise ValueError("bad k or clip percentile")
    return c


def quantize_weights_outliers_raw(w_ptr: int, n: int, k: int, clip_percentile: float, q_ptr: int, s_ptr: int,
                                  idx_ptr: int, val_ptr: int, cap: int, stream: int = 0) -> int:
    return int(library().qw_quantize_weights_outliers(w_ptr, n, k, float(clip_percentile), q_ptr, s_ptr, idx_ptr,
                                                      val_ptr, cap, stream))


def w8a16_gemm_outliers_raw(x_ptr: int, q_ptr: int, s_ptr: int, idx_ptr: int, val_ptr: int, cap: int, y_ptr: int,
                            m: int, n: int, k: int, stream: int = 0, path: int = 0) -> int:
    return int(library().qw_w8a16_gemm_outliers_path(x_ptr, q_ptr, s_ptr, idx_ptr, val_ptr, cap, y_ptr, m, n, k,
                                                     int(path), stream))


def w8a16_gemm_tile_raw(x_ptr: int, q_ptr: int, s_ptr: int, z_ptr: int, idx_ptr: int, val_ptr: int, cap: int,
                        y_ptr: int, m: int, n: int, k: int, tile: int, stream: int = 0) -> int:
    return int(library().qw_w8a16_gemm_tile(x_ptr, q_ptr, s_ptr, z_ptr, idx_ptr, val_ptr, cap, y_ptr, m, n, k,
                                            int(tile), stream))


def w8a8_gemm_tile_raw(qx_ptr: int, sx_ptr: int, q_ptr: int, s_ptr: int, y_ptr: int, m: int, n: int, k: int,
                       tile: int, stream: int = 0) -> int:
    return int(library().qw_w8a8_gemm_tile(qx_ptr, sx_ptr, q_ptr, s_ptr, y_ptr, m, n, k, int(tile), stream))


def quantize_weights_asym_raw(w_ptr: int, n: int, k: int, q_ptr: int, s_ptr: int, z_ptr: int,
                              stream: int = 0) -> int:
    return int(library().qw_quantize_weights_asym(w_ptr, n, k, q_ptr, s_ptr, z_ptr, stream))


def w8a16_gemm_asym_raw(x_ptr: int, q_ptr: int, s_ptr: int, z_ptr: int, y_ptr: int, m: int, n: int, k: int,
                        stream: int = 0, path: int = 0) -> int:
    return int(library().qw_w8a16_gemm_asym_path(x_ptr, q_ptr, s_ptr, z_ptr, y_ptr, m, n, k, int(path), stream))


def w8a16_gemm_raw(x_ptr: int, q_ptr: int, s_ptr: int, y_ptr: int, m: int, n: int, k: int,
                   stream: int = 0, path: int = 0) -> int:
    return int(library().qw_w8a16_gemm_path(x_ptr, q_ptr, s_ptr, y_ptr, m, n, k, int(path), stream))


def w8a8_gemm_raw(qx_ptr: int, sx_ptr: int, q_ptr: int, s_ptr: int, y_ptr: int, m: int, n: int,
                  k: int, stream: int = 0, path: int = 0) -> int:
    return int(library().qw_w8a8_gemm_path(qx_ptr, sx_ptr, q_ptr, s_ptr, y_ptr, m, n, k, int(path), stream))


# ---------------------------------------------------------------------------
# torch-facing calls
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_of(t) -> int:
    torch = _torch()
    return int(torch.cuda.current_stream(t.device).cuda_stream)


def _check(t, name, dtype, shape=None, ndim=None, device=None):
    """Validate one tensor argument before its pointer reaches the library:
    a torch.Tensor of `dtype`, contiguous, with exactly `shape` (or `ndim`
    dimensions), on `device`.  The C ABI cannot see sizes or devices, so
    every check that protects a kernel from reading or writing outside a
    buffer happens here."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if device is not None and t.device != device:
        raise ValueError("%s must be on %s (the device of the first operand), got %s" % (name, device, t.device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must be %d-D, got shape %s" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _require_gpu(t, name):
    """The first tensor operand fixes the device; it must be a GPU tensor."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device, got %s" % (name, t.device))
    return t.device


def _outputs(out, specs, device):
    """Check caller-provided outputs (a tensor or a tuple of tensors) against
    (name, dtype, shape) specs; None means 'allocate them'."""
    torch = _torch()
    if out is None:
        return tuple(torch.empty(shape, dtype=dtype, device=device) for _, dtype, shape in specs)
    outs = out if isinstance(out, (tuple, list)) else (out,)
    if len(outs) != len(specs):
        raise ValueError("out must hold %d tensor(s), got %d" % (len(specs), len(outs)))
    for t, (name, dtype, shape) in zip(outs, specs):
        _check(t, name, dtype, shape=shape, device=device)
    return tuple(outs)


def _check_path(path):
    if path not in PATHS:
        raise ValueError("path must be one of %s" % sorted(PATHS))


# Validation of each call, separate from the launch so that every rejection
# can be exercised without a GPU (with tensors on one device of any type).

def _validate_quantize(w, out, device):
    torch = _torch()
    f16 = isinstance(w, torch.Tensor) and w.dtype == torch.float16
    _check(w, "w", torch.float16 if f16 else torch.float32, ndim=2, device=device)
    n, k = w.shape
    q, s = _outputs(out, (("q", torch.int8, (n, k)), ("scales", torch.float16, (n,))), device)
    return f16, n, k, q, s


def _validate_gemm(x, q, scales, out, path, device, zeros=None, ol=None, a8=False, sx=None):
    torch = _torch()
    _check(x, "qx" if a8 else "x", torch.int8 if a8 else torch.float16, ndim=2, device=device)
    m, k = x.shape
    _check(q, "q", torch.int8, ndim=2, device=device)
    n = q.shape[0]
    _check(q, "q", torch.int8, shape=(n, k), device=device)
    _check(scales, "scales", torch.float16, shape=(n,), device=device)
    if sx is not None:
        _check(sx, "sx", torch.float16, shape=(m,), device=device)
    if zeros is not None:
        _check(zeros, "zeros", torch.int8, shape=(n,), device=device)
    cap = 0
    if ol is not None:
        ol_idx, ol_val = ol
        _check(ol_idx, "ol_idx", torch.int32, ndim=2, device=device)
        cap = ol_idx.shape[1]
        _check(ol_idx, "ol_idx", torch.int32, shape=(n, cap), device=device)
        _check(ol_val, "ol_val", torch.float32, shape=(n, cap), device=device)
    if path is not None:
        _check_path(path)
    (y,) = _outputs(out, (("out", torch.float16, (m, n)),), device)
    return m, n, k, cap, y


def quantize_weights(w, clip_percentile: float = 100.0, out=None):
    """Per-output-row symmetric int8 quantization of a Linear weight.

    w: cuda float32 or float16 [N, K] (K % 16 == 0, K <= 65536; fp16 is
    widened exactly to fp32 first).  clip_percentile in (0, 100]; 100 uses
    the row absmax.  Returns (q int8 [N, K], scales float16 [N]);
    ``out=(q, scales)`` writes into preallocated tensors.
    """
    device = _require_gpu(w, "w")
    f16, n, k, q, s = _validate_quantize(w, out, device)
    raw = quantize_weights_f16_raw if f16 else quantize_weights_raw
    st = raw(w.data_ptr(), n, k, clip_percentile, q.data_ptr(), s.data_ptr(), _stream_of(w))
    if st != QW_SUCCESS:
        raise QwError(st, "qw_quantize_weights_f16" if f16 else "qw_quantize_weights")
    return q, s


def w8a16_gemm(x, q, scales, out=None, path: str = "auto"):
    """Y = X * dequant(q)^T: x cuda fp16 [M, K], q int8 [N, K], scales fp16 [N]
    -> fp16 [M, N].  ``path`` forces a kernel ("gemv", "skinny" or "mfma")."""
    device = _require_gpu(x, "x")
    m, n, k, _, y = _validate_gemm(x, q, scales, out, path, device)
    st = w8a16_gemm_raw(x.data_ptr(), q.data_ptr(), scales.data_ptr(), y.data_ptr(), m, n, k,
                        _stream_of(x), PATHS[path])
    if st != QW_SUCCESS:
        raise QwError(st, "qw_w8a16_gemm")
    return y


def w8a16_gemm_tune(x, q, scales, out=None):
    """Time every kernel and MFMA tile for this shape on these buffers,
    record the fastest for the shape's bucket, and return Y (the winner's
    result).  Later automatic calls of the bucket use the record."""
    device = _require_gpu(x, "x")
    m, n, k, _, y = _validate_gemm(x, q, scales, out, None, device)
    st = w8a16_gemm_tune_raw(x.data_ptr(), q.data_ptr(), scales.data_ptr(), y.data_ptr(), m, n, k, _stream_of(x))
    if st != QW_SUCCESS:
        raise QwError(st, "qw_w8a16_gemm_tune")
    return y


def _validate_fixed_range(w, bounds, out, device):
    torch = _torch()
    _check(w, "w", torch.float32, ndim=2, device=device)
    n, k = w.shape
    _check(bounds, "bounds", torch.float32, shape=(n,), device=device)
    q, s = _outputs(out, (("q", torch.int8, (n, k)), ("scales", torch.float16, (n,))), device)
    return n, k, q, s


def quantize_weights_fixed_range(w, bounds, out=None):
    """Per-row symmetric int8 quantization with given clip bounds: w cuda
    float32 [N, K], bounds cuda float32 [N] (finite, >= 0).  Returns
    (q int8 [N, K], scales float16 [N])."""
    device = _require_gpu(w, "w")
    n, k, q, s = _validate_fixed_range(w, bounds, out, device)
    st = quantize_weights_fixed_range_raw(w.data_ptr(), n, k, bounds.data_ptr(), q.data_ptr(), s.data_ptr(),
                                          _stream_of(w))
    if st != QW_SUCCESS:
        raise QwError(st, "qw_quantize_weights_fixed_range")
    return q, s


def quantize_weights_outliers(w, clip_percentile: float):
    """Outlier-aware quantization of a cuda float32 [N, K] weight: returns
    (q int8 [N, K], scales float16 [N], ol_idx int32 [N, C], ol_val float32
    [N, C]) with C = outlier_capacity(K, clip_percentile)."""
    torch = _torch()
    device = _require_gpu(w, "w")
    _check(w, "w", torch.float32, ndim=2, device=device)
    n, k = w.shape
    cap = outlier_capacity(k, clip_percentile)
    q = torch.empty((n, k), dtype=torch.int8, device=device)
    s = torch.empty((n,), dtype=torch.float16, device=device)
    # (at least one slot allocated, so that the pointers are valid with cap 0)
    idx = torch.empty((n, max(cap, 1)), dtype=torch.int32, device=device)[:, :cap]
    val = torch.empty((n, max(cap, 1)), dtype=torch.float32, device=device)[:, :cap]
    st = quantize_weights_outliers_raw(w.data_ptr(), n, k, clip_percentile, q.data_ptr(), s.data_ptr(),
                                       idx.data_ptr(), val.data_ptr(), cap, _stream_of(w))
    if st != QW_SUCCESS:
        raise QwError(st, "qw_quantize_weights_outliers")
    return q, s, idx, val


def w8a16_gemm_outliers(x, q, scales, ol_idx, ol_val, out=None, path: str = "auto"):
    """Y = X * dequant(q)^T plus the exact outlier side lists: x cuda fp16
    [M, K], q int8 [N, K], scales fp16 [N], ol_idx int32 [N, C], ol_val
    float32 [N, C] -> fp16 [M, N]."""
    device = _require_gpu(x, "x")
    m, n, k, cap, y = _validate_gemm(x, q, scales, out, path, device, ol=(ol_idx, ol_val))
    st = w8a16_gemm_outliers_raw(x.data_ptr(), q.data_ptr(), scales.data_ptr(), ol_idx.data_ptr(),
                                 ol_val.data_ptr(), cap, y.data_ptr(), m, n, k, _stream_of(x), PATHS[path])
    if st != QW_SUCCESS:
        raise QwError(st, "qw_w8a16_gemm_outliers")
    return y


def w8a16_gemm_tile(x, q, scales, tile, zeros=None, outliers=None, out=None):
    """The MFMA GEMM with a given output tile (BN, BM), one of MFMA_TILES:
    what w8a16_gemm (no zeros, no outliers), w8a16_gemm_asym (zeros int8
    [N]) or w8a16_gemm_outliers (outliers = (ol_idx, ol_val)) computes."""
    if tuple(tile) not in MFMA_TILES:
        raise ValueError("tile must be one of %s, got %r" % (MFMA_TILES, tile))
    if zeros is not None and outliers is not None:
        raise ValueError("outlier side lists belong to symmetric codes: pass zeros or outliers, not both")
    device = _require_gpu(x, "x")
    m, n, k, cap, y = _validate_gemm(x, q, scales, out, None, device, zeros=zeros, ol=outliers)
    idx_ptr = outliers[0].data_ptr() if outliers is not None else None
    val_ptr = outliers[1].data_ptr() if outliers is not None else None
    st = w8a16_gemm_tile_raw(x.data_ptr(), q.data_ptr(), scales.data_ptr(),
                             zeros.data_ptr() if zeros is not None else None, idx_ptr, val_ptr, cap,
                             y.data_ptr(), m, n, k, tile[0] * 1000 + tile[1], _stream_of(x))
    if st != QW_SUCCESS:
        raise QwError(st, "qw_w8a16_gemm_tile")
    return y


def quantize_weights_asym(w, out=None):
    """Asymmetric per-row int8 quantization of a cuda float32 [N, K] weight:
    returns (q int8 [N, K], scales float16 [N], zeros int8 [N]) with
    W ~ scales[:, None] * (q - zeros[:, None])."""
    torch = _torch()
    device = _require_gpu(w, "w")
    _check(w, "w", torch.float32, ndim=2, device=device)
    n, k = w.shape
    q, s, z = _outputs(out, (("q", torch.int8, (n, k)), ("scales", torch.float16, (n,)),
                             ("zeros", torch.int8, (n,))), device)
    st = quantize_weights_asym_raw(w.data_ptr(), n, k, q.data_ptr(), s.data_ptr(), z.data_ptr(), _stream_of(w))
    if st != QW_SUCCESS:
        raise QwError(st, "qw_quantize_weights_asym")
    return q, s, z


def w8a16_gemm_asym(x, q, scales, zeros, out=None, path: str = "auto"):
    """Y = X * (scales * (q - zeros))^T for asymmetric weights: x cuda fp16
    [M, K], q int8 [N, K], scales fp16 [N], zeros int8 [N] -> fp16 [M, N]."""
    device = _require_gpu(x, "x")
    m, n, k, _, y = _validate_gemm(x, q, scales, out, path, device, zeros=zeros)
    st = w8a16_gemm_asym_raw(x.data_ptr(), q.data_ptr(), scales.data_ptr(), zeros.data_ptr(), y.data_ptr(),
                             m, n, k, _stream_of(x), PATHS[path])
    if st != QW_SUCCESS:
        raise QwError(st, "qw_w8a16_gemm_asym")
    return y


def quantize_activations(x, out=None):
    """Per-token (per-row) symmetric int8 quantization of fp16 activations
    [M, K] for W8A8: the weights' quantizer with the row absmax.  Returns
    (qx int8 [M, K], sx float16 [M])."""
    return quantize_weights(x, 100.0, out=out)


def w8a8_gemm(qx, sx, q, scales, out=None):
    """Y = (qx * q^T) * sx[:, None] * scales[None, :]: qx int8 [M, K], sx fp16
    [M], q int8 [N, K], scales fp16 [N] -> fp16 [M, N]."""
    device = _require_gpu(qx, "qx")
    m, n, k, _, y = _validate_gemm(qx, q, scales, out, None, device, a8=True, sx=sx)
    st = w8a8_gemm_raw(qx.data_ptr(), sx.data_ptr(), q.data_ptr(), scales.data_ptr(), y.data_ptr(),
                       m, n, k, _stream_of(qx))
    if st != QW_SUCCESS:
        raise QwError(st, "qw_w8a8_gemm")
    return y


def w8a8_gemm_tile(qx, sx, q, scales, tile, out=None):
    """The W8A8 MFMA GEMM with a given output tile (BN, BM), one of
    W8A8_TILES; otherwise as w8a8_gemm."""
    if tuple(tile) not in W8A8_TILES:
        raise ValueError("tile must be one of %s, got %r" % (W8A8_TILES, tile))
    device = _require_gpu(qx, "qx")
    m, n, k, _, y = _validate_gemm(qx, q, scales, out, None, device, a8=True, sx=sx)
    st = w8a8_gemm_tile_raw(qx.data_ptr(), sx.data_ptr(), q.data_ptr(), scales.data_ptr(), y.data_ptr(),
                            m, n, k, tile[0] * 1000 + tile[1], _stream_of(qx))
    if st != QW_SUCCESS:
        raise QwError(st, "qw_w8a8_gemm_tile")
    return y


def probe_stream_read_raw(p: int, nbytes: int, magic: int, sink_ptr: int, stream: int = 0) -> int:
    """Enqueue the plain streaming-read probe over nbytes at device pointer p."""
    return int(library().qw_probe_stream_read(p, nbytes, magic & 0xffffffff, sink_ptr, stream))


def probe_shader_clock_raw(out_ptr: int, stream: int = 0) -> int:
    """Enqueue the shader-clock probe; out_ptr: two uint64 of device memory."""
    return int(library().qw_probe_shader_clock(out_ptr, stream))


__all__ = ["quantize_weights", "quantize_weights_fixed_range", "quantize_weights_asym", "w8a16_gemm_asym",
           "quantize_weights_outliers", "w8a16_gemm_outliers", "outlier_capacity",
           "w8a16_gemm_tune", "tuned_choice", "tune_reset", "w8a16_gemm_tune_raw",
           "quantize_activations", "w8a16_gemm", "w8a8_gemm", "QwError",
           "status_string", "version", "library", "auto_path", "mfma_tile", "w8a8_tile",
           "quantize_weights_raw", "quantize_weights_f16_raw", "quantize_weights_fixed_range_raw", "quantize_weights_asym_raw", "w8a16_gemm_asym_raw",
           "quantize_weights_outliers_raw", "w8a16_gemm_outliers_raw", "w8a16_gemm_raw", "w8a8_gemm_raw",
           "probe_stream_read_raw", "probe_shader_clock_raw", "PATHS", "LIBRARY_PATH"]

"""Helpers for the GPU parity tests: move seeded host buffers to the device,
call the library through its C ABI, bring results back, and compare with the
oracle on exactly the same host buffers."""

from __future__ import annotations

import sys

import numpy as np

TOL_REL = 2e-3
TOL_ABS = 1e-3


def say(msg: str):
    """Name the case before each GPU step (flushed, so it survives a crash)."""
    print("[gpu] " + msg, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def dev(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t) -> np.ndarray:
    torch = torch_mod()
    torch.cuda.synchronize()
    return t.cpu().numpy()


def gpu_quantize(w: np.ndarray, pct: float):
    """Quantize fp32 or fp16 weights on the GPU through the C ABI; returns
    (q int8, scale bits uint16)."""
    import int8_weight_quantized_amd as qw
    torch = torch_mod()
    n, k = w.shape
    wd = dev(w)
    qd = torch.full((n, k), 99, dtype=torch.int8, device="cuda:0")
    sd = torch.full((n,), 0x5555, dtype=torch.int16, device="cuda:0")
    raw = qw.quantize_weights_f16_raw if w.dtype == np.float16 else qw.quantize_weights_raw
    st = raw(wd.data_ptr(), n, k, pct, qd.data_ptr(), sd.data_ptr(),
             int(torch.cuda.current_stream().cuda_stream))
    assert st == 0, qw.status_string(st)
    return host(qd), host(sd).view(np.uint16)


def gpu_quantize_fixed(w: np.ndarray, bounds: np.ndarray):
    """Fixed-range quantization on the GPU through the C ABI; returns
    (q int8, scale bits uint16)."""
    import int8_weight_quantized_amd as qw
    torch = torch_mod()
    n, k = w.shape
    wd = dev(np.ascontiguousarray(w, dtype=np.float32))
    bd = dev(np.ascontiguousarray(bounds, dtype=np.float32))
    qd = torch.full((n, k), 99, dtype=torch.int8, device="cuda:0")
    sd = torch.full((n,), 0x5555, dtype=torch.int16, device="cuda:0")
    st = qw.quantize_weights_fixed_range_raw(wd.data_ptr(), n, k, bd.data_ptr(), qd.data_ptr(), sd.data_ptr(),
                                             int(torch.cuda.current_stream().cuda_stream))
    assert st == 0, qw.status_string(st)
    return host(qd), host(sd).view(np.uint16)


def gpu_gemm(x: np.ndarray, q: np.ndarray, s_bits: np.ndarray, path: int = 0):
    """W8A16 GEMM on the GPU through the C ABI; returns Y as float16."""
    import int8_weight_quantized_amd as qw
    torch = torch_mod()
    m, k = x.shape
    n = q.shape[0]
    xd = dev(np.ascontiguousarray(x, dtype=np.float16).view(np.int16))
    qd = dev(q)
    sd = dev(np.ascontiguousarray(s_bits, dtype=np.uint16).view(np.int16))
    yd = torch.full((m, n), 0x7e00, dtype=torch.int16, device="cuda:0")  # NaN canary
    st = qw.w8a16_gemm_raw(xd.data_ptr(), qd.data_ptr(), sd.data_ptr(), yd.data_ptr(), m, n, k,
                           int(torch.cuda.current_stream().cuda_stream), path)
    assert st == 0, qw.status_string(st)
    return host(yd).view(np.float16)


def gpu_w8a8(qx: np.ndarray, sx_bits: np.ndarray, q: np.ndarray, s_bits: np.ndarray, path: int = 0):
    """W8A8 GEMM on the GPU through the C ABI; returns Y as float16."""
    import int8_weight_quantized_amd as qw
    torch = torch_mod()
    m, k = qx.shape
    n = q.shape[0]
    qxd = dev(np.ascontiguousarray(qx, dtype=np.int8))
    sxd = dev(np.ascontiguousarray(sx_bits, dtype=np.uint16).view(np.int16))
    qd = dev(np.ascontiguousarray(q, dtype=np.int8))
    sd = dev(np.ascontiguousarray(s_bits, dtype=np.uint16).view(np.int16))
    yd = torch.full((m, n), 0x7e00, dtype=torch.int16, device="cuda:0")  # NaN canary
    st = qw.w8a8_gemm_raw(qxd.data_ptr(), sxd.data_ptr(), qd.data_ptr(), sd.data_ptr(), yd.data_ptr(),
                          m, n, k, int(torch.cuda.current_stream().cuda_stream), path)
    assert st == 0, qw.status_string(st)
    return host(yd).view(np.float16)


def assert_w8a8_close(y: np.ndarray, ref: np.ndarray, what: str = ""):
    """Element-wise |Y - ref| <= 2^-10 |ref| + 2^-24: one binary16 rounding
    (at most 2^-11 relative) of a value carrying at most two binary32
    roundings, with the binary16 subnormal quantum covered by 2^-24."""
    y64 = y.astype(np.float64)
    assert np.all(np.isfinite(y64)), "%s: non-finite output" % what
    bound = np.abs(ref) * 2.0 ** -10 + 2.0 ** -24
    bad = np.argwhere(np.abs(y64 - ref) > bound)
    assert bad.size == 0, "%s: %d elements out of bound, first %s (gpu %r, ref %r)" % (
        what, len(bad), bad[0], y64[tuple(bad[0])], ref[tuple(bad[0])])


def assert_gemm_close(y: np.ndarray, ref: np.ndarray, what: str = ""):
    """max |Y - ref| <= 2e-3 * max|ref| + 1e-3, with ref the binary64 oracle."""
    y64 = y.astype(np.float64)
    assert np.all(np.isfinite(y64)), "%s: non-finite output" % what
    err = np.abs(y64 - ref).max() if ref.size else 0.0
    tol = TOL_REL * (np.abs(ref).max() if ref.size else 0.0) + TOL_ABS
    assert err <= tol, "%s: max err %.3g > tol %.3g" % (what, err, tol)
    return err, tol


def gpu_gemm_tile(x: np.ndarray, q: np.ndarray, s_bits: np.ndarray, tile, zeros=None, idx=None, val=None):
    """The MFMA GEMM with a forced output tile (BN, BM) through the C ABI
    (zeros: asymmetric codes; idx/val: outlier side lists); returns Y as
    float16."""
    import int8_weight_quantized_amd as qw
    torch = torch_mod()
    m, k = x.shape
    n = q.shape[0]
    xd = dev(np.ascontiguousarray(x, dtype=np.float16).view(np.int16))
    qd = dev(np.ascontiguousarray(q, dtype=np.int8))
    sd = dev(np.ascontiguousarray(s_bits, dtype=np.uint16).view(np.int16))
    zd = dev(np.ascontiguousarray(zeros, dtype=np.int8)) if zeros is not None else None
    cap = idx.shape[1] if idx is not None else 0
    idd = dev(np.ascontiguousarray(idx, dtype=np.int32)) if cap else None
    vd = dev(np.ascontiguousarray(val, dtype=np.float32)) if cap else None
    yd = torch.full((m, n), 0x7e00, dtype=torch.int16, device="cuda:0")  # NaN canary
    st = qw.w8a16_gemm_tile_raw(xd.data_ptr(), qd.data_ptr(), sd.data_ptr(),
                                zd.data_ptr() if zd is not None else None,
                                idd.data_ptr() if idd is not None else None,
                                vd.data_ptr() if vd is not None else None, cap, yd.data_ptr(), m, n, k,
                                tile[0] * 1000 + tile[1], int(torch.cuda.current_stream().cuda_stream))
    assert st == 0, qw.status_string(st)
    return host(yd).view(np.float16)


def gpu_w8a8_tile(qx: np.ndarray, sx_bits: np.ndarray, q: np.ndarray, s_bits: np.ndarray, tile):
    """W8A8 MFMA GEMM with a forced output tile (BN, BM) through the C ABI;
    returns Y as float16."""
    import int8_weight_quantized_amd as qw
    torch = torch_mod()
    m, k = qx.shape
    n = q.shape[0]
    qxd = dev(np.ascontiguousarray(qx, dtype=np.int8))
    sxd = dev(np.ascontiguousarray(sx_bits, dtype=np.uint16).view(np.int16))
    qd = dev(np.ascontiguousarray(q, dtype=np.int8))
    sd = dev(np.ascontiguousarray(s_bits, dtype=np.uint16).view(np.int16))
    yd = torch.full((m, n), 0x7e00, dtype=torch.int16, device="cuda:0")  # NaN canary
    st = qw.w8a8_gemm_tile_raw(qxd.data_ptr(), sxd.data_ptr(), qd.data_ptr(), sd.data_ptr(), yd.data_ptr(),
                               m, n, k, tile[0] * 1000 + tile[1], int(torch.cuda.current_stream().cuda_stream))
    assert st == 0, qw.status_string(st)
    return host(yd).view(np.float16)

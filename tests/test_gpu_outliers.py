"""GPU parity of the outlier-aware path (dense int8 inliers plus exact side
lists of the elements above the clip bound) through the C ABI against the
CPU oracle on the same seeded host buffers.

  * quantizer: codes, fp16 scale bits, side-list columns and values
    bit-identical;
  * GEMM: max |Y - ref| <= 2e-3 * max|ref| + 1e-3 on every kernel path and
    every MFMA tile, bit-exact where the arithmetic is exact in fp32.
"""

import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import assert_gemm_close, dev, host, say, torch_mod

pytestmark = pytest.mark.gpu

GEMV, MFMA, SKINNY = 1, 2, 3


def gpu_quantize_outliers(w, pct, cap=None):
    import int8_weight_quantized_amd as qw
    torch = torch_mod()
    n, k = w.shape
    if cap is None:
        cap = qw.outlier_capacity(k, pct)
    wd = dev(np.ascontiguousarray(w, dtype=np.float32))
    qd = torch.full((n, k), 99, dtype=torch.int8, device="cuda:0")
    sd = torch.full((n,), 0x5555, dtype=torch.int16, device="cuda:0")
    idd = torch.full((n, max(cap, 1)), 12345, dtype=torch.int32, device="cuda:0")
    vd = torch.full((n, max(cap, 1)), 7.0, dtype=torch.float32, device="cuda:0")
    st = qw.quantize_weights_outliers_raw(wd.data_ptr(), n, k, pct, qd.data_ptr(), sd.data_ptr(), idd.data_ptr(),
                                          vd.data_ptr(), cap, int(torch.cuda.current_stream().cuda_stream))
    assert st == 0, qw.status_string(st)
    return host(qd), host(sd).view(np.uint16), host(idd)[:, :cap], host(vd)[:, :cap]


def gpu_gemm_outliers(x, q, s_bits, idx, val, path=0):
    import int8_weight_quantized_amd as qw
    torch = torch_mod()
    m, k = x.shape
    n = q.shape[0]
    cap = idx.shape[1]
    xd = dev(np.ascontiguousarray(x, dtype=np.float16).view(np.int16))
    qd = dev(np.ascontiguousarray(q, dtype=np.int8))
    sd = dev(np.ascontiguousarray(s_bits, dtype=np.uint16).view(np.int16))
    idd = dev(np.ascontiguousarray(idx if cap else np.zeros((n, 1)), dtype=np.int32))
    vd = dev(np.ascontiguousarray(val if cap else np.zeros((n, 1)), dtype=np.float32))
    yd = torch.full((m, n), 0x7e00, dtype=torch.int16, device="cuda:0")  # NaN canary
    st = qw.w8a16_gemm_outliers_raw(xd.data_ptr(), qd.data_ptr(), sd.data_ptr(), idd.data_ptr(), vd.data_ptr(),
                                    cap, yd.data_ptr(), m, n, k, int(torch.cuda.current_stream().cuda_stream), path)
    assert st == 0, qw.status_string(st)
    return host(yd).view(np.float16)


def _weights(n, k, seed, frac=0.001):
    """Gaussian weights with planted outliers (GOBO-style), some rows with
    several of them, one all-zero row."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    hit = rng.choice(n * k, size=max(2, int(round(frac * n * k))), replace=False)
    w.flat[hit] = (rng.standard_normal(hit.size) * 0.2).astype(np.float32)
    w[min(1, n - 1), : min(k, 3)] = np.float32([0.9, -0.8, 0.7][: min(k, 3)])
    w[n // 2] = 0.0
    return w


@pytest.mark.parametrize("n,k,pct", [(64, 1024, 99.99), (37, 1040, 99.9), (96, 4096, 99.9), (300, 1024, 99.0),
                                     (17, 64, 90.0), (8, 4112, 99.99), (5, 65536, 99.999), (40, 256, 100.0)])
def test_quantize_outliers(n, k, pct):
    w = _weights(n, k, n * 17 + k)
    say("quantize outliers n=%d k=%d pct=%r" % (n, k, pct))
    q_ref, s_ref, i_ref, v_ref = oracle.quantize_outliers(w, pct)
    q, s, idx, val = gpu_quantize_outliers(w, pct)
    assert np.array_equal(s, s_ref), "scales differ at rows %s" % np.nonzero(s != s_ref)[0][:5]
    assert np.array_equal(idx, i_ref), "side-list columns differ at rows %s" % np.nonzero((idx != i_ref).any(1))[0][:5]
    assert np.array_equal(val.view(np.uint32), v_ref.view(np.uint32)), "side-list values differ"
    assert np.array_equal(q, q_ref), "codes differ at %s" % np.argwhere(q != q_ref)[:5]


def test_quantize_outliers_wider_than_needed():
    """More slots than the capacity: the extra ones are written -1 / 0."""
    w = _weights(20, 1024, 3)
    say("quantize outliers cap=6 n=20 k=1024")
    q_ref, s_ref, i_ref, v_ref = oracle.quantize_outliers(w, 99.99, cap=6)
    q, s, idx, val = gpu_quantize_outliers(w, 99.99, cap=6)
    assert np.array_equal(idx, i_ref) and np.array_equal(val, v_ref) and np.array_equal(q, q_ref)


SHAPES = [(1, 1000, 272, 99.9), (2, 300, 2064, 99.9), (8, 517, 2064, 99.99), (17, 300, 528, 99.0),
          (65, 130, 96, 95.0), (130, 260, 4112, 99.9), (300, 513, 1040, 99.99), (257, 129, 144, 97.0),
          (20, 260, 2064, 99.9)]


@pytest.mark.parametrize("m,n,k,pct", SHAPES)
def test_gemm_outliers_every_path(m, n, k, pct):
    import int8_weight_quantized_amd as qw
    x = synthetic.random_x(m, k, m + n)
    w = _weights(n, k, m * 5 + n, frac=0.003)
    q, s, idx, val = oracle.quantize_outliers(w, pct)
    ref = oracle.gemm_outliers(x, q, s, idx, val)
    for path in (0, GEMV, SKINNY, MFMA):
        if path == GEMV and m > 8:
            continue
        if path == MFMA and idx.shape[1] > 4:
            continue
        say("gemm outliers path=%d m=%d n=%d k=%d cap=%d" % (path, m, n, k, idx.shape[1]))
        assert_gemm_close(gpu_gemm_outliers(x, q, s, idx, val, path), ref,
                          "outliers path %d %dx%dx%d cap %d" % (path, m, n, k, idx.shape[1]))
    assert qw.outlier_capacity(k, pct) == idx.shape[1]


# every MFMA tile with side lists (the 256 x 128 tile runs as 256 x 64)
TILE_SHAPES = [(512, 27392, 256), (2048, 4608, 128), (256, 27392, 128), (384, 13824, 128), (96, 27392, 256),
               (129, 40960, 64)]


def test_gemm_outliers_mfma_tiles():
    for m, n, k in TILE_SHAPES:
        x = synthetic.random_x(m, k, m + 3)
        w = _weights(n, k, n + 11, frac=0.002)
        q, s, idx, val = oracle.quantize_outliers(w, 99.5, cap=4)
        say("gemm outliers mfma m=%d n=%d k=%d" % (m, n, k))
        y = gpu_gemm_outliers(x, q, s, idx, val, MFMA)
        rng = np.random.default_rng(m + n)
        mr = np.unique(np.r_[0, m - 1, rng.integers(0, m, 4)])
        nc = np.unique(np.r_[0, n - 1, rng.integers(0, n, 4), np.nonzero(idx[:, 0] >= 0)[0][:8]])
        mi = np.concatenate([np.repeat(mr, n), np.tile(np.arange(m), len(nc)), rng.integers(0, m, 4096)])
        ni = np.concatenate([np.tile(np.arange(n), len(mr)), np.repeat(nc, m), rng.integers(0, n, 4096)])
        assert_gemm_close(y[mi, ni], oracle.gemm_outliers_sampled(x, q, s, idx, val, mi, ni),
                          "outliers mfma %dx%dx%d (sampled)" % (m, n, k))
        assert np.all(np.isfinite(y.astype(np.float32)))


# Every 4-wave MFMA tile forced, with side lists of one to four slots per
# row, rows of 512 and 1024 codes (the FFN's), ragged m and n: against the
# oracle, and bit-exact on exact inputs.
FORCED_TILES = [(256, 128), (256, 64), (128, 128), (128, 64)]


@pytest.mark.parametrize("tile", FORCED_TILES)
@pytest.mark.parametrize("m,n,k,cap", [(300, 520, 1024, 1), (97, 333, 512, 3), (256, 256, 1024, 3)])
def test_gemm_outliers_forced_tiles(tile, m, n, k, cap):
    from gpu_util import gpu_gemm_tile
    x = synthetic.random_x(m, k, m + k + cap)
    w = _weights(n, k, n + k + cap, frac=0.003)
    pct = 99.99 if cap == 1 else 99.7
    q, s, idx, val = oracle.quantize_outliers(w, pct, cap=max(cap, oracle.outlier_capacity(k, pct)))
    idx, val = np.ascontiguousarray(idx), np.ascontiguousarray(val)
    say("gemm outliers forced tile=%s m=%d n=%d k=%d cap=%d" % (tile, m, n, k, idx.shape[1]))
    y = gpu_gemm_tile(x, q, s, tile, idx=idx, val=val)
    assert_gemm_close(y, oracle.gemm_outliers(x, q, s, idx, val), "outliers forced tile %s %dx%dx%d" % (tile, m, n, k))
    # the automatic MFMA tile on the same data
    y_auto = gpu_gemm_outliers(x, q, s, idx, val, MFMA)
    assert np.all(np.isfinite(y.astype(np.float32)))
    assert_gemm_close(y, y_auto.astype(np.float64), "forced tile vs auto %s" % (tile,))


@pytest.mark.parametrize("tile", FORCED_TILES)
def test_gemm_outliers_forced_tiles_exact(tile):
    """Exact arithmetic (as below) through the forced tiles at k = 1024 and
    512: bit-exact against the oracle."""
    from gpu_util import gpu_gemm_tile
    for (m, n, k) in ((130, 300, 1024), (64, 64, 512)):
        rng = np.random.default_rng(m + n + k + tile[0] + tile[1])
        x = rng.integers(-1, 2, size=(m, k)).astype(np.float16)
        q = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
        e = rng.integers(0, 11, size=n)
        s = (2.0 ** (-e)).astype(np.float16)
        cap = 4
        idx = np.full((n, cap), -1, dtype=np.int32)
        val = np.zeros((n, cap), dtype=np.float32)
        for r in range(n):
            c = int(rng.integers(0, cap + 1))
            cols = np.sort(rng.choice(k, size=c, replace=False))
            idx[r, :c] = cols
            val[r, :c] = rng.integers(-4000, 4000, size=c) * (float(s[r]) / 8)
            q[r, cols] = 0
        say("gemm outliers forced tile exact tile=%s m=%d n=%d k=%d" % (tile, m, n, k))
        y = gpu_gemm_tile(x, q, s.view(np.uint16), tile, idx=idx, val=val)
        want = oracle.f64_to_f16_bits(oracle.gemm_outliers(x, q, s.view(np.uint16), idx, val))
        assert np.array_equal(y.view(np.uint16), want), (tile, m, n, k)


@pytest.mark.parametrize("path", [GEMV, SKINNY, MFMA])
@pytest.mark.parametrize("m,n,k", [(1, 96, 512), (8, 130, 2048), (200, 300, 1040), (20, 25000, 2064)])
def test_gemm_outliers_exact_arithmetic_bitexact(path, m, n, k):
    """X in {-1,0,1}, power-of-two scales, outlier values that are multiples
    of S / 8 (so value / S is exact too): every step is exact in fp32, and
    Y is bit-exact."""
    if path == GEMV and m > 8:
        pytest.skip("the GEMV kernel takes m <= 8")
    rng = np.random.default_rng(m + n + k + path)
    x = rng.integers(-1, 2, size=(m, k)).astype(np.float16)
    q = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    e = rng.integers(0, 11, size=n)
    s = (2.0 ** (-e)).astype(np.float16)
    cap = 4
    idx = np.full((n, cap), -1, dtype=np.int32)
    val = np.zeros((n, cap), dtype=np.float32)
    for r in range(n):
        c = int(rng.integers(0, cap + 1))
        cols = np.sort(rng.choice(k, size=c, replace=False))
        idx[r, :c] = cols
        val[r, :c] = rng.integers(-4000, 4000, size=c) * (float(s[r]) / 8)
        q[r, cols] = 0
    say("gemm outliers exact path=%d m=%d n=%d k=%d" % (path, m, n, k))
    y = gpu_gemm_outliers(x, q, s.view(np.uint16), idx, val, path)
    want = oracle.f64_to_f16_bits(oracle.gemm_outliers(x, q, s.view(np.uint16), idx, val))
    assert np.array_equal(y.view(np.uint16), want)


def test_outlier_workload_end_to_end():
    """The Transformer-big FFN workload with its 0.1% outliers: quantize with
    side lists, multiply; the result matches the oracle and sits closer to
    the unquantized product than clipping alone."""
    wl = synthetic.BY_NAME["transformer_big_ffn_outliers_m4096_k1024_n4096"]
    x, w = synthetic.make_inputs(wl)
    say("quantize outliers %s" % wl.name)
    q, s, idx, val = gpu_quantize_outliers(w, wl.clip_percentile)
    q_ref, s_ref, i_ref, v_ref = oracle.quantize_outliers(w, wl.clip_percentile)
    assert np.array_equal(q, q_ref) and np.array_equal(s, s_ref) and np.array_equal(idx, i_ref)
    assert np.array_equal(val, v_ref)
    say("gemm outliers %s" % wl.name)
    y = gpu_gemm_outliers(x, q, s, idx, val)
    # every output against the binary64 oracle
    assert_gemm_close(y, oracle.gemm_outliers(x, q, s, idx, val), "ffn outliers")
    rng = np.random.default_rng(7)
    mi = np.concatenate([np.repeat([0, 777, 4095], wl.n), rng.integers(0, wl.m, 8192)])
    ni = np.concatenate([np.tile(np.arange(wl.n), 3), rng.integers(0, wl.n, 8192)])
    # against the unquantized product on sampled outputs
    exact = np.einsum("ck,ck->c", x[mi].astype(np.float64), w[ni].astype(np.float64))
    qc, sc, _ = oracle.quantize(w, wl.clip_percentile)
    clipped = oracle.gemm_sampled(x, qc, sc, mi, ni)
    err_ol = np.abs(y[mi, ni].astype(np.float64) - exact).mean()
    err_clip = np.abs(clipped - exact).mean()
    assert err_ol < err_clip, (err_ol, err_clip)

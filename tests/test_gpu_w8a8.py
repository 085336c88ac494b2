"""GPU parity of the W8A8 (int8 x int8) GEMM through the C ABI against the CPU
oracle on the same seeded host buffers.

The activation codes and scales come from quantizing each activation row
with the weights' quantizer (the fp16-input entry point with the row
absmax); they must equal the oracle's bit for bit before the matmul is
compared.  The matmul bound is element-wise: |Y - ref| <= 2^-10 |ref| +
2^-24 (one binary16 rounding of a value with at most two binary32
roundings); with power-of-two scales and |acc| < 2^24 every step is exact
and Y must be bit-exact.
"""

import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import assert_w8a8_close, gpu_quantize, gpu_w8a8, gpu_w8a8_tile, say

pytestmark = pytest.mark.gpu


def _codes(m, n, k, seed):
    x = synthetic.random_x(m, k, seed)
    w = synthetic.random_w(n, k, seed + 1)
    qx, sx, _ = oracle.quantize(x.astype(np.float32), 100.0)
    q, s, _ = oracle.quantize(w, 100.0)
    return qx, sx, q, s


def _sample_indices(m, n, rng, rows=6, cols=6, points=4096):
    # whole output rows, whole output columns, scattered points
    mr = np.unique(np.r_[0, m - 1, rng.integers(0, m, rows)])
    nc = np.unique(np.r_[0, n - 1, rng.integers(0, n, cols)])
    mi = np.concatenate([np.repeat(mr, n), np.tile(np.arange(m), len(nc)), rng.integers(0, m, points)])
    ni = np.concatenate([np.tile(np.arange(n), len(mr)), np.repeat(nc, m), rng.integers(0, n, points)])
    return mi, ni


@pytest.mark.parametrize("name", ["small_batch_m8_k4096_n4608", "chatglm2_prefill_m512_k4096_n27392",
                                  "transformer_big_ffn_outliers_m4096_k1024_n4096"])
def test_w8a8_workload(name):
    wl = synthetic.BY_NAME[name]
    x, w = synthetic.make_inputs(wl)
    q, s, _ = oracle.quantize(w, wl.clip_percentile)
    qx_ref, sx_ref, _ = oracle.quantize(x.astype(np.float32), 100.0)
    say("w8a8 activation quantize %s m=%d k=%d" % (name, wl.m, wl.k))
    qx, sx = gpu_quantize(x, 100.0)
    assert np.array_equal(sx, sx_ref) and np.array_equal(qx, qx_ref)
    say("w8a8 gemm %s m=%d n=%d k=%d" % (name, wl.m, wl.n, wl.k))
    y = gpu_w8a8(qx, sx, q, s)
    if wl.m * wl.n * wl.k <= 4e8:
        assert_w8a8_close(y, oracle.w8a8_gemm(qx, sx, q, s), name)
    else:
        mi, ni = _sample_indices(wl.m, wl.n, np.random.default_rng(321))
        assert_w8a8_close(y[mi, ni], oracle.w8a8_gemm_sampled(qx, sx, q, s, mi, ni), name + " (sampled)")
        assert np.all(np.isfinite(y.astype(np.float32))), "non-finite output outside the sample"


# ragged m, n and k across several tiles of every tile shape
SHAPES = [(1, 1000, 272), (3, 257, 528), (4, 64, 16), (8, 517, 2064), (9, 200, 272), (17, 300, 528),
          (31, 129, 80), (64, 256, 256), (65, 130, 96), (100, 390, 656), (128, 128, 4096),
          (130, 260, 4112), (257, 129, 144), (300, 513, 1040), (129, 600, 528), (70, 72, 16400),
          (24, 300, 2064), (32, 1200, 4112), (20, 25000, 2064),
          (24, 13000, 2064)]  # the last four: 32-row skinny passes


MFMA, SKINNY = 2, 3


# Grids on a tile with 256 weight rows whose tile order walks several
# weight-tile columns per group, the last group narrower; whole outputs.
@pytest.mark.parametrize("m,n,k", [(512, 27392, 64), (4096, 3328, 64), (8192, 4352, 64)])
def test_w8a8_grouped_tile_order(m, n, k):
    import int8_weight_quantized_amd as qw
    assert qw.w8a8_tile(m, n, k)[0] == 256
    qx, sx, q, s = _codes(m, n, k, seed=m + n + 9)
    say("w8a8 gemm mfma grouped order m=%d n=%d k=%d" % (m, n, k))
    ref = oracle.w8a8_gemm(qx, sx, q, s)
    assert_w8a8_close(gpu_w8a8(qx, sx, q, s, MFMA), ref, "w8a8 grouped order %dx%dx%d" % (m, n, k))
    # the 256 x 128 tile on the same grids (the automatic choice gives them
    # the ping-pong tile)
    say("w8a8 gemm mfma 256x128 grouped order m=%d n=%d k=%d" % (m, n, k))
    assert_w8a8_close(gpu_w8a8_tile(qx, sx, q, s, (256, 128)), ref, "w8a8 256x128 grouped %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("path", [0, SKINNY, MFMA])
@pytest.mark.parametrize("m,n,k", SHAPES)
def test_w8a8_shapes(m, n, k, path):
    qx, sx, q, s = _codes(m, n, k, seed=m * 1000 + n)
    say("w8a8 gemm path=%d m=%d n=%d k=%d" % (path, m, n, k))
    assert_w8a8_close(gpu_w8a8(qx, sx, q, s, path), oracle.w8a8_gemm(qx, sx, q, s),
                      "w8a8 path %d %dx%dx%d" % (path, m, n, k))


TILE_SHAPES = [(512, 27392, 256), (2048, 4608, 128), (256, 27392, 128), (384, 13824, 128),
               (96, 27392, 256), (1024, 9216, 128), (4096, 4096, 64), (320, 6144, 144),
               (384, 32768, 128), (129, 40960, 64), (200, 16384, 80), (1088, 9216, 128)]


def test_w8a8_every_tile_shape():
    import int8_weight_quantized_amd as qw
    seen = set()
    for m, n, k in TILE_SHAPES:
        tile = qw.w8a8_tile(m, n, k)
        seen.add(tile)
        qx, sx, q, s = _codes(m, n, k, seed=m + n)
        say("w8a8 gemm tile=%s m=%d n=%d k=%d" % (tile, m, n, k))
        y = gpu_w8a8(qx, sx, q, s)
        mi, ni = _sample_indices(m, n, np.random.default_rng(m * 7 + n))
        assert_w8a8_close(y[mi, ni], oracle.w8a8_gemm_sampled(qx, sx, q, s, mi, ni),
                          "w8a8 tile %s %dx%dx%d (sampled)" % (tile, m, n, k))
        assert np.all(np.isfinite(y.astype(np.float32))), "non-finite output outside the sample"
    # the W8A8 kernel has four tile shapes (no 128 x 128)
    assert seen == {(256, 256), (256, 128), (256, 64), (128, 64)}, "tiles exercised: %s" % sorted(seen)


@pytest.mark.parametrize("path", [SKINNY, MFMA])
@pytest.mark.parametrize("m,n,k", [(1, 96, 512), (8, 130, 1040), (100, 390, 1040), (640, 4100, 272)])
def test_w8a8_exact_arithmetic_bitexact(m, n, k, path):
    """|acc| <= k * 127^2 < 2^24 for k <= 1040 and power-of-two scales: every
    step is exact in binary32, so Y is the binary16 rounding of the exact
    value, bit for bit."""
    rng = np.random.default_rng(m + n + k)
    qx = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    q = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    # Sx * S in [2^-21, 2^-10]: the largest |Y| (2^24 * 2^-10) stays finite in
    # binary16 and the smallest reach its subnormal range
    sx = (2.0 ** (-rng.integers(0, 8, size=m))).astype(np.float16).view(np.uint16)
    s = (2.0 ** (-rng.integers(10, 15, size=n))).astype(np.float16).view(np.uint16)
    # saturate one row and one column so |acc| reaches k * 127^2
    qx[0, :] = 127
    q[0, :] = 127
    say("w8a8 exact path=%d m=%d n=%d k=%d" % (path, m, n, k))
    y = gpu_w8a8(qx, sx, q, s, path)
    want = oracle.f64_to_f16_bits(oracle.w8a8_gemm(qx, sx, q, s))
    assert np.array_equal(y.view(np.uint16), want)


def test_w8a8_longest_k_saturated():
    """k at the documented maximum with saturated codes: |acc| = k * 127^2 =
    2^17 * 16129 sits just below 2^31, so the int32 accumulator must not
    wrap; 16129 * 2^17 is exact in binary32, so Y is bit-exact."""
    import int8_weight_quantized_amd as qw
    k = 131072
    rng = np.random.default_rng(17)
    qx = np.empty((3, k), dtype=np.int8)
    qx[0], qx[1] = 127, -127
    qx[2] = rng.integers(-127, 128, size=k)
    q = np.empty((4, k), dtype=np.int8)
    q[0], q[1] = 127, -127
    q[2:] = rng.integers(-127, 128, size=(2, k))
    sx = np.full(3, np.float16(2.0 ** -8)).view(np.uint16)
    s = np.full(4, np.float16(2.0 ** -9)).view(np.uint16)
    want = oracle.f64_to_f16_bits(oracle.w8a8_gemm(qx, sx, q, s))
    for path in (SKINNY, MFMA):
        say("w8a8 longest k path=%d m=3 n=4 k=%d" % (path, k))
        y = gpu_w8a8(qx, sx, q, s, path)
        assert np.array_equal(y.view(np.uint16), want)
    assert qw.w8a8_gemm_raw(1 << 20, 2 << 20, 3 << 20, 4 << 20, 5 << 20, 1, 4, k + 16) == qw.QW_ERROR_UNSUPPORTED


def test_w8a8_zero_codes_and_zero_scales():
    m, n, k = 70, 300, 272
    qx, sx, q, s = _codes(m, n, k, seed=5)
    qx[3] = 0
    sx[5] = 0
    q[7] = 0
    s[11] = 0
    say("w8a8 zero rows m=%d n=%d k=%d" % (m, n, k))
    y = gpu_w8a8(qx, sx, q, s, MFMA)
    bits = y.view(np.uint16)
    # all-zero codes give an exact integer 0, so +0; a zero scale gives a
    # zero of either sign (the MFMA epilogue rounds the product to fp16 in
    # one fused step, which writes +0 for a negative sum times 0)
    assert np.all(bits[3, :] == 0) and np.all(bits[:, 7] == 0), "zero codes must give +0"
    assert np.all(y[5, :] == 0) and np.all(y[:, 11] == 0), "zero scale must give zero"
    y2 = gpu_w8a8(qx, sx, q, s, SKINNY)
    assert np.all(y2[5, :] == 0) and np.all(y2[:, 11] == 0)
    assert_w8a8_close(y, oracle.w8a8_gemm(qx, sx, q, s), "w8a8 zero rows")


def test_w8a8_deterministic():
    qx, sx, q, s = _codes(512, 4608, 1024, seed=9)
    say("w8a8 determinism")
    a = gpu_w8a8(qx, sx, q, s)
    b = gpu_w8a8(qx, sx, q, s)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_w8a8_torch_binding():
    torch = pytest.importorskip("torch")
    import int8_weight_quantized_amd as qw
    m, n, k = 96, 520, 528
    x = synthetic.random_x(m, k, 11)
    w = synthetic.random_w(n, k, 12)
    say("w8a8 torch binding m=%d n=%d k=%d" % (m, n, k))
    xd = torch.from_numpy(x).to("cuda:0")
    q, s = qw.quantize_weights(torch.from_numpy(w).to("cuda:0"))
    qx, sx = qw.quantize_activations(xd)
    y = qw.w8a8_gemm(qx, sx, q, s)
    torch.cuda.synchronize()
    ref = oracle.w8a8_gemm(qx.cpu().numpy(), sx.cpu().numpy().view(np.uint16), q.cpu().numpy(),
                           s.cpu().numpy().view(np.uint16))
    assert_w8a8_close(y.cpu().numpy(), ref, "torch binding")

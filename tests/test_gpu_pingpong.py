"""GPU parity of the 256 x 256 ping-pong MFMA tile (8 waves, two wave groups
taking turns at the matrix cores, three LDS stages), forced through
qw_w8a16_gemm_tile / qw_w8a8_gemm_tile and reached through the automatic
kernel choice.

Cases span one to several tiles with ragged tails in m (the second wave
group's rows partly or wholly past m), n (partial weight tiles, rows not a
multiple of 8) and k (a last k step of 16 to 48 codes), the shortest k
(one partial step), k steps of 1 to 5 (every tail of the unrolled loop),
asymmetric codes, outlier side lists (1 to 4 slots), exact arithmetic
(bit-exact), and grids whose tile order walks several groups of weight-tile
columns with a narrower last group.  The oracle is the binary64 CPU
implementation on the same host buffers; tolerance as for every W8A16 path.
"""

import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import assert_gemm_close, assert_w8a8_close, gpu_gemm, gpu_gemm_tile, gpu_w8a8_tile, say

pytestmark = pytest.mark.gpu

PP = (256, 256)
MFMA = 2


def _case(m, n, k, seed):
    x = synthetic.random_x(m, k, seed)
    w = synthetic.random_w(n, k, seed + 1)
    q, s, _ = oracle.quantize(w, 100.0)
    return x, q, s


# k = 16 ... 320: one partial step, then 1-5 full steps (the unrolled loop's
# every tail); the others cross several tiles with ragged m, n and k
SHAPES = [
    (256, 256, 16), (256, 256, 64), (256, 256, 128), (256, 256, 192), (256, 512, 256), (256, 256, 320),
    (1, 256, 64), (129, 300, 336), (257, 300, 16), (300, 522, 1040), (513, 1000, 4112), (700, 777, 2064),
    (128, 4104, 1024),
]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_pingpong_shapes(m, n, k):
    x, q, s = _case(m, n, k, seed=3 * m + n + k)
    say("gemm pingpong m=%d n=%d k=%d" % (m, n, k))
    y = gpu_gemm_tile(x, q, s, PP)
    assert_gemm_close(y, oracle.gemm(x, q, s), "pingpong %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("m,n,k", [(256, 256, 64), (300, 522, 1040), (512, 600, 4096)])
def test_pingpong_exact_arithmetic_bitexact(m, n, k):
    """X in {-2..2}, power-of-two scales: every partial sum is exact in fp32,
    so Y is the fp16 rounding of the exact value, bit for bit."""
    rng = np.random.default_rng(m + n + k)
    x = rng.integers(-2, 3, size=(m, k)).astype(np.float16)
    q = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    s = (2.0 ** (-rng.integers(0, 11, size=n))).astype(np.float16).view(np.uint16)
    say("gemm pingpong exact m=%d n=%d k=%d" % (m, n, k))
    y = gpu_gemm_tile(x, q, s, PP)
    assert np.array_equal(y.view(np.uint16), oracle.f64_to_f16_bits(oracle.gemm(x, q, s)))


@pytest.mark.parametrize("m,n,k", [(256, 256, 64), (300, 522, 1040), (513, 300, 336)])
def test_pingpong_asym(m, n, k):
    x = synthetic.random_x(m, k, m + 7)
    w = synthetic.random_w(n, k, n + 9)
    q, s, z = oracle.quantize_asym(w)
    say("gemm pingpong asym m=%d n=%d k=%d" % (m, n, k))
    y = gpu_gemm_tile(x, q, s, PP, zeros=z)
    assert_gemm_close(y, oracle.gemm_asym(x, q, s, z), "pingpong asym %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("m,n,k", [(256, 256, 64), (300, 522, 1040)])
def test_pingpong_asym_exact_arithmetic_bitexact(m, n, k):
    rng = np.random.default_rng(m * 3 + n + k)
    x = rng.integers(-2, 3, size=(m, k)).astype(np.float16)
    q = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    z = rng.integers(-20, 21, size=n).astype(np.int8)
    s = (2.0 ** (-rng.integers(0, 11, size=n))).astype(np.float16).view(np.uint16)
    say("gemm pingpong asym exact m=%d n=%d k=%d" % (m, n, k))
    y = gpu_gemm_tile(x, q, s, PP, zeros=z)
    assert np.array_equal(y.view(np.uint16), oracle.f64_to_f16_bits(oracle.gemm_asym(x, q, s, z)))


def _outlier_weights(n, k, seed, frac=0.002):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    hit = rng.choice(n * k, size=max(2, int(round(frac * n * k))), replace=False)
    w.flat[hit] = (rng.standard_normal(hit.size) * 0.2).astype(np.float32)
    w[n // 2] = 0.0
    return w


# (the percentile sets the slots per row: k - 1 - floor(pct / 100 (k - 1)))
@pytest.mark.parametrize("m,n,k,pct,cap", [(256, 256, 64, 99.5, 1), (300, 522, 1040, 99.7, 4),
                                           (513, 300, 2064, 99.9, 3)])
def test_pingpong_outliers(m, n, k, pct, cap):
    x = synthetic.random_x(m, k, m + 5)
    w = _outlier_weights(n, k, n + k)
    assert oracle.outlier_capacity(k, pct) == cap
    q, s, idx, val = oracle.quantize_outliers(w, pct, cap=cap)
    say("gemm pingpong outliers m=%d n=%d k=%d cap=%d" % (m, n, k, cap))
    y = gpu_gemm_tile(x, q, s, PP, idx=idx, val=val)
    assert_gemm_close(y, oracle.gemm_outliers(x, q, s, idx, val), "pingpong outliers %dx%dx%d" % (m, n, k))


def test_pingpong_outliers_exact_arithmetic_bitexact():
    """Outlier values that are multiples of S / 8 (value / S exact): Y is
    bit-exact."""
    m, n, k, cap = 300, 522, 1040, 4
    rng = np.random.default_rng(11)
    x = rng.integers(-1, 2, size=(m, k)).astype(np.float16)
    q = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    s = (2.0 ** (-rng.integers(0, 11, size=n))).astype(np.float16)
    idx = np.full((n, cap), -1, dtype=np.int32)
    val = np.zeros((n, cap), dtype=np.float32)
    for r in range(n):
        c = int(rng.integers(0, cap + 1))
        cols = np.sort(rng.choice(k, size=c, replace=False))
        idx[r, :c] = cols
        val[r, :c] = rng.integers(-4000, 4000, size=c) * (float(s[r]) / 8)
        q[r, cols] = 0
    say("gemm pingpong outliers exact m=%d n=%d k=%d" % (m, n, k))
    y = gpu_gemm_tile(x, q, s.view(np.uint16), PP, idx=idx, val=val)
    want = oracle.f64_to_f16_bits(oracle.gemm_outliers(x, q, s.view(np.uint16), idx, val))
    assert np.array_equal(y.view(np.uint16), want)


# Grids whose tile order walks several weight-tile column groups with a
# narrower last group: 107 columns in groups of 14, 13 in groups of 7, 17
# over several rounds of resident tiles.  The whole output is compared.
GROUPED = [(512, 27392, 64), (4096, 3328, 64), (8192, 4352, 64)]


@pytest.mark.parametrize("m,n,k", GROUPED)
def test_pingpong_grouped_tile_order(m, n, k):
    import int8_weight_quantized_amd as qw
    assert qw.mfma_tile(m, n, k) == PP
    x, q, s = _case(m, n, k, seed=m + n)
    say("gemm pingpong grouped m=%d n=%d k=%d" % (m, n, k))
    y = gpu_gemm(x, q, s, path=MFMA)
    assert_gemm_close(y, oracle.gemm(x, q, s), "pingpong grouped %dx%dx%d" % (m, n, k))


def test_pingpong_choice():
    """The automatic choice: the prefill and FFN shapes take the ping-pong
    tile; 256 rows on 27392 channels (107 tiles, under half the CUs), 384
    rows (a third more rows than whole 64-row tiles) and 129 rows do not;
    nor does a k beyond the tile's limit."""
    import int8_weight_quantized_amd as qw
    assert qw.mfma_tile(512, 27392, 4096) == PP
    assert qw.mfma_tile(4096, 4096, 1024) == PP
    assert qw.mfma_tile(2048, 4608, 4096) == PP
    assert qw.mfma_tile(256, 27392, 4096) != PP
    assert qw.mfma_tile(384, 27392, 4096) != PP
    assert qw.mfma_tile(129, 40960, 4096) != PP
    assert qw.mfma_tile(512, 27392, qw.PINGPONG_MAX_K + 16) != PP



# ---- W8A8 (int8 activation codes, v_mfma_i32_32x32x32_i8) ----

def _codes(m, n, k, seed):
    x = synthetic.random_x(m, k, seed)
    w = synthetic.random_w(n, k, seed + 1)
    qx, sx, _ = oracle.quantize(x.astype(np.float32), 100.0)
    q, s, _ = oracle.quantize(w, 100.0)
    return qx, sx, q, s


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_pingpong_w8a8_shapes(m, n, k):
    qx, sx, q, s = _codes(m, n, k, seed=5 * m + n + k)
    say("w8a8 pingpong m=%d n=%d k=%d" % (m, n, k))
    y = gpu_w8a8_tile(qx, sx, q, s, PP)
    assert_w8a8_close(y, oracle.w8a8_gemm(qx, sx, q, s), "w8a8 pingpong %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("m,n,k", [(256, 256, 64), (300, 522, 1040), (640, 4100, 272)])
def test_pingpong_w8a8_exact_arithmetic_bitexact(m, n, k):
    """|acc| <= k * 127^2 < 2^24 and power-of-two scales: Y is the binary16
    rounding of the exact value, bit for bit (one row and one column
    saturated)."""
    rng = np.random.default_rng(m + 2 * n + k)
    qx = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    q = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    sx = (2.0 ** (-rng.integers(0, 8, size=m))).astype(np.float16).view(np.uint16)
    s = (2.0 ** (-rng.integers(10, 15, size=n))).astype(np.float16).view(np.uint16)
    qx[0, :] = 127
    q[0, :] = 127
    say("w8a8 pingpong exact m=%d n=%d k=%d" % (m, n, k))
    y = gpu_w8a8_tile(qx, sx, q, s, PP)
    assert np.array_equal(y.view(np.uint16), oracle.f64_to_f16_bits(oracle.w8a8_gemm(qx, sx, q, s)))


@pytest.mark.parametrize("m,n,k", [(512, 27392, 64), (4096, 3328, 64)])
def test_pingpong_w8a8_grouped_tile_order(m, n, k):
    qx, sx, q, s = _codes(m, n, k, seed=m + n + 1)
    say("w8a8 pingpong grouped m=%d n=%d k=%d" % (m, n, k))
    y = gpu_w8a8_tile(qx, sx, q, s, PP)
    assert_w8a8_close(y, oracle.w8a8_gemm(qx, sx, q, s), "w8a8 pingpong grouped %dx%dx%d" % (m, n, k))

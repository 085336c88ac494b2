"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same
seeded host buffers.

  * quantizer: int8 codes and fp16 scale bits must be identical (bit-exact);
  * GEMM: max |Y - ref| <= 2e-3 * max|ref| + 1e-3 against the binary64
    oracle computed from the same (already bit-identical) codes and scales;
    the exact-arithmetic case must be bit-exact.

Full workload sizes run in the launch configuration the benchmark times
(the automatic kernel choice), every output compared; forced-path sweeps
over other shapes compare whole output rows, whole output columns and
scattered points, computed one by one.
"""

import functools

import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import assert_gemm_close, gpu_gemm, gpu_gemm_tile, gpu_quantize, say

pytestmark = pytest.mark.gpu

GEMV, MFMA, SKINNY = 1, 2, 3


@functools.lru_cache(maxsize=2)
def workload_data(name):
    wl = synthetic.BY_NAME[name]
    x, w = synthetic.make_inputs(wl)
    q, s, t = oracle.quantize(w, wl.clip_percentile)
    return wl, x, w, q, s


NAMES = [w.name for w in synthetic.WORKLOADS]


@pytest.mark.parametrize("name", NAMES)
def test_quantize_workload_bitexact(name):
    wl, x, w, q_ref, s_ref = workload_data(name)
    say("quantize %s n=%d k=%d pct=%g" % (name, wl.n, wl.k, wl.clip_percentile))
    q, s = gpu_quantize(w, wl.clip_percentile)
    bad_s = np.nonzero(s != s_ref)[0]
    assert bad_s.size == 0, "scale mismatch rows %s gpu %s oracle %s" % (bad_s[:5], s[bad_s[:5]], s_ref[bad_s[:5]])
    bad = np.argwhere(q != q_ref)
    assert bad.size == 0, "code mismatch at %s" % (bad[:5],)


def _sample_indices(m, n, rng, rows=6, cols=6, points=4096):
    # whole output rows, whole output columns, scattered points
    mr = np.unique(np.r_[0, m - 1, rng.integers(0, m, rows)])
    mi = [np.repeat(mr, n)]
    ni = [np.tile(np.arange(n), len(mr))]
    nc = np.unique(np.r_[0, n - 1, rng.integers(0, n, cols)])
    mi.append(np.tile(np.arange(m), len(nc)))
    ni.append(np.repeat(nc, m))
    mi.append(rng.integers(0, m, points))
    ni.append(rng.integers(0, n, points))
    return np.concatenate(mi), np.concatenate(ni)


@pytest.mark.parametrize("name", NAMES)
def test_gemm_workload(name):
    """Every workload at full size through the automatic kernel choice (the
    launch configuration the benchmark times), every output compared with
    the binary64 oracle (the prefill one is about 10^11 multiply-adds on
    the host's OpenMP threads)."""
    wl, x, w, q, s = workload_data(name)
    say("gemm auto %s m=%d n=%d k=%d" % (name, wl.m, wl.n, wl.k))
    y = gpu_gemm(x, q, s)
    ref = oracle.gemm(x, q, s)
    assert_gemm_close(y, ref, name)


# Shapes that between them land on every MFMA tile shape (the choice depends
# on the CU count and the kernels' occupancy, so coverage is checked, not
# which shape gets which tile).
TILE_SHAPES = [(512, 27392, 256), (2048, 4608, 128), (256, 27392, 128), (384, 13824, 128),
               (96, 27392, 256), (1024, 9216, 128), (4096, 4096, 64), (320, 6144, 144),
               (384, 32768, 128), (129, 40960, 64), (1088, 9216, 128)]


def test_mfma_every_tile_shape():
    import int8_weight_quantized_amd as qw
    seen = set()
    for m, n, k in TILE_SHAPES:
        tile = qw.mfma_tile(m, n, k)
        seen.add(tile)
        x, q, s = _small_case(m, n, k, seed=m + n)
        say("gemm mfma tile=%s m=%d n=%d k=%d" % (tile, m, n, k))
        y = gpu_gemm(x, q, s, path=MFMA)
        mi, ni = _sample_indices(m, n, np.random.default_rng(m * 7 + n))
        ref = oracle.gemm_sampled(x, q, s, mi, ni)
        assert_gemm_close(y[mi, ni], ref, "mfma tile %s %dx%dx%d (sampled)" % (tile, m, n, k))
        assert np.all(np.isfinite(y.astype(np.float32))), "non-finite output outside the sample"
    assert seen == {(256, 256), (256, 128), (256, 64), (128, 128), (128, 64)}, "tiles exercised: %s" % sorted(seen)


# Grids on the 256 x 128 tile (forced: the automatic choice gives these
# shapes the 256 x 256 ping-pong tile) whose tile order walks several
# weight-tile columns per group, the last group narrower: 107 and 13
# columns with every tile of an XCD resident at once, 17 columns over
# several rounds of resident tiles.  The whole output is compared.
GROUPED_SHAPES = [(512, 27392, 64), (4096, 3328, 64), (8192, 4352, 64)]


@pytest.mark.parametrize("m,n,k", GROUPED_SHAPES)
def test_mfma_grouped_tile_order(m, n, k):
    x, q, s = _small_case(m, n, k, seed=m + n + 5)
    say("gemm mfma 256x128 grouped order m=%d n=%d k=%d" % (m, n, k))
    y = gpu_gemm_tile(x, q, s, (256, 128))
    assert_gemm_close(y, oracle.gemm(x, q, s), "mfma grouped order %dx%dx%d" % (m, n, k))


# Shapes spanning several tiles with ragged tails in m, n and k.
SMALL_SHAPES = [
    (1, 1000, 272), (1, 129, 1040), (2, 300, 2064), (3, 257, 528), (4, 64, 16),
    (5, 77, 4096), (7, 130, 1024), (8, 517, 2064), (4, 33, 4112),
]
MFMA_SHAPES = SMALL_SHAPES + [
    (9, 200, 272), (16, 128, 64), (17, 300, 528), (31, 129, 80), (33, 257, 1024),
    (64, 256, 256), (65, 130, 96), (100, 390, 656), (128, 128, 4096), (130, 260, 4112),
    (257, 129, 144), (300, 513, 1040), (129, 600, 528), (256, 1024, 336),
]


def _small_case(m, n, k, seed):
    x = synthetic.random_x(m, k, seed)
    w = synthetic.random_w(n, k, seed + 1)
    q, s, _ = oracle.quantize(w, 100.0)
    return x, q, s


@pytest.mark.parametrize("m,n,k", SMALL_SHAPES)
def test_gemv_small_shapes(m, n, k):
    x, q, s = _small_case(m, n, k, seed=m * 1000 + n)
    say("gemm gemv m=%d n=%d k=%d" % (m, n, k))
    y = gpu_gemm(x, q, s, path=GEMV)
    assert_gemm_close(y, oracle.gemm(x, q, s), "gemv %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("m,n,k", MFMA_SHAPES)
def test_skinny_small_shapes(m, n, k):
    x, q, s = _small_case(m, n, k, seed=m * 1000 + n + 7)
    say("gemm skinny m=%d n=%d k=%d" % (m, n, k))
    y = gpu_gemm(x, q, s, path=SKINNY)
    assert_gemm_close(y, oracle.gemm(x, q, s), "skinny %dx%dx%d" % (m, n, k))


# The skinny kernel with two 16-row activation tiles per wave (17..32 rows,
# k >= 2048) and with one (more rows, or shorter k), at weight shapes that
# select several of its k splits; n = 27392, 25000 and 13000 take four
# weight tiles per workgroup, the last of them partly past n.
SKINNY_TILE_SHAPES = [(32, 4608, 4096), (24, 27392, 2048), (32, 27392, 4096), (20, 25000, 2064), (24, 13000, 2064), (17, 1000, 2064), (31, 130, 4096), (24, 600, 1024),
                      (64, 4608, 4096), (48, 2048, 64), (40, 4096, 8192), (64, 65536, 64), (100, 1200, 2064)]


@pytest.mark.parametrize("m,n,k", SKINNY_TILE_SHAPES)
def test_skinny_activation_tiles(m, n, k):
    x, q, s = _small_case(m, n, k, seed=m * 7 + n)
    say("gemm skinny tiles m=%d n=%d k=%d" % (m, n, k))
    y = gpu_gemm(x, q, s, path=SKINNY)
    assert_gemm_close(y, oracle.gemm(x, q, s), "skinny tiles %dx%dx%d" % (m, n, k))


# Long rows: k beyond what the GEMV stages in LDS (it then falls back to the
# skinny kernel), and long reductions on every path.
LONG_K_SHAPES = [(1, 64, 65536), (2, 40, 32784), (9, 72, 16400), (70, 72, 16400)]


@pytest.mark.parametrize("m,n,k", LONG_K_SHAPES)
def test_gemm_long_k(m, n, k):
    x, q, s = _small_case(m, n, k, seed=7 * m + n)
    say("gemm long-k auto m=%d n=%d k=%d" % (m, n, k))
    y = gpu_gemm(x, q, s)
    assert_gemm_close(y, oracle.gemm(x, q, s), "long-k auto %dx%dx%d" % (m, n, k))
    for path in (SKINNY, MFMA):
        say("gemm long-k path=%d m=%d n=%d k=%d" % (path, m, n, k))
        y = gpu_gemm(x, q, s, path=path)
        assert_gemm_close(y, oracle.gemm(x, q, s), "long-k path %d %dx%dx%d" % (path, m, n, k))


def test_gemm_rows_beyond_mfma_limit():
    """k = QW_MFMA_MAX_K + 16 with 65 activation rows, where the MFMA
    kernel would otherwise run: the automatic choice takes the skinny kernel
    (64-bit indexing); sampled outputs against the oracle."""
    import int8_weight_quantized_amd as qw
    m, n, k = 65, 16, qw.MFMA_MAX_K + 16
    assert qw.auto_path(m, n, k) == "skinny"
    x, q, s = _small_case(m, n, k, seed=11)
    say("gemm auto beyond the MFMA row limit m=%d n=%d k=%d" % (m, n, k))
    y = gpu_gemm(x, q, s)
    rng = np.random.default_rng(5)
    mi = np.r_[0, m - 1, 16, 64, rng.integers(0, m, 28)]
    ni = np.r_[0, n - 1, 15, 8, rng.integers(0, n, 28)]
    assert_gemm_close(y[mi, ni], oracle.gemm_sampled(x, q, s, mi, ni), "k beyond the MFMA limit (sampled)")


@pytest.mark.parametrize("m,n,k", MFMA_SHAPES)
def test_mfma_small_shapes(m, n, k):
    x, q, s = _small_case(m, n, k, seed=m * 1000 + n)
    say("gemm mfma m=%d n=%d k=%d" % (m, n, k))
    y = gpu_gemm(x, q, s, path=MFMA)
    assert_gemm_close(y, oracle.gemm(x, q, s), "mfma %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("path", [GEMV, SKINNY, MFMA])
@pytest.mark.parametrize("m,n,k", [(1, 96, 512), (4, 200, 1024), (8, 130, 2048)])
def test_gemm_exact_arithmetic_bitexact(path, m, n, k):
    """X in {-1,0,1}, power-of-two scales: every partial sum is exact in fp32,
    so Y must be the fp16 rounding of the exact value, bit for bit."""
    rng = np.random.default_rng(m + n + k)
    x = rng.integers(-1, 2, size=(m, k)).astype(np.float16)
    q = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    e = rng.integers(0, 11, size=n)
    s = (2.0 ** (-e)).astype(np.float16).view(np.uint16)
    say("gemm exact path=%d m=%d n=%d k=%d" % (path, m, n, k))
    y = gpu_gemm(x, q, s, path=path)
    want = oracle.f64_to_f16_bits(oracle.gemm(x, q, s))
    assert np.array_equal(y.view(np.uint16), want)


@pytest.mark.parametrize("m", [1, 2, 4, 8])
def test_paths_agree_with_oracle_at_same_m(m):
    wl = synthetic.BY_NAME["small_batch_m8_k4096_n4608"]
    x = synthetic.random_x(m, wl.k, 77)
    _, _, _, q, s = workload_data(wl.name)
    ref = oracle.gemm(x, q, s)
    for path in (GEMV, SKINNY, MFMA):
        say("gemm path=%d m=%d n=%d k=%d" % (path, m, wl.n, wl.k))
        assert_gemm_close(gpu_gemm(x, q, s, path=path), ref, "path %d m %d" % (path, m))


def test_gemm_deterministic():
    wl, x, w, q, s = workload_data("small_batch_m8_k4096_n4608")
    say("gemm determinism")
    for path in (GEMV, SKINNY, MFMA):
        a = gpu_gemm(x, q, s, path=path)
        b = gpu_gemm(x, q, s, path=path)
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_gemm_zero_activation_and_zero_rows():
    rng = np.random.default_rng(5)
    m, n, k = 5, 70, 320
    w = synthetic.random_w(n, k, 9)
    w[3] = 0.0
    q, s, _ = oracle.quantize(w, 100.0)
    x = rng.standard_normal((m, k)).astype(np.float16)
    x[2] = 0.0
    for path in (GEMV, SKINNY, MFMA):
        say("gemm zeros path=%d" % path)
        y = gpu_gemm(x, q, s, path=path)
        assert np.all(y[2].view(np.uint16) == 0) and np.all(y[:, 3].view(np.uint16) == 0)
        assert_gemm_close(y, oracle.gemm(x, q, s), "zeros")


# ---------------------------------------------------------------------------
# quantizer edge cases
# ---------------------------------------------------------------------------

def _check_quant(w, pct, what):
    say("quantize %s n=%d k=%d pct=%r" % (what, w.shape[0], w.shape[1], pct))
    q_ref, s_ref, _ = oracle.quantize(w, pct)
    q, s = gpu_quantize(w, pct)
    assert np.array_equal(s, s_ref), "%s: scales differ at rows %s" % (what, np.nonzero(s != s_ref)[0][:5])
    assert np.array_equal(q, q_ref), "%s: codes differ at %s" % (what, np.argwhere(q != q_ref)[:5])


def test_quantize_degenerate_rows():
    k = 64
    w = np.zeros((8, k), dtype=np.float32)
    w[1, 5] = -3.0e-3
    w[2, :] = 7.0e-2
    w[3, :4] = np.float32(1e-9)          # scale underflows fp16 -> 0
    w[4, :] = np.float32(2.0**-10)       # subnormal fp16 scale
    w[4, ::3] = -np.float32(3 * 2.0**-12)
    w[5, 0] = np.float32(1.0e7)          # scale overflows fp16 -> inf, codes 0
    w[5, 1] = np.float32(1.0)
    w[6, :] = -0.0                       # negative zeros
    w[7, :] = np.float32(1.5e-41)        # binary32 subnormal weights
    for pct in (100.0, 99.0, 50.0, 1.0):
        _check_quant(w, pct, "degenerate")


def test_quantize_exact_ties():
    """Weights exactly on (j + 1/2) * S: round-half-to-even decides."""
    js = np.arange(-127, 127, dtype=np.float64)
    rows = []
    for sv in (0.000634, 0.0009766, 0.00047, 0.0008):
        s16 = float(np.float16(sv))
        row = np.concatenate([(js + 0.5) * s16, [127.0 * s16], np.zeros(17)]).astype(np.float32)
        rows.append(row)
    _check_quant(np.stack(rows), 100.0, "ties")


@pytest.mark.parametrize("k", [16, 32, 1040, 4096 + 16, 16384, 65536])
@pytest.mark.parametrize("pct", [100.0, 99.99, 90.0, 50.0, 0.5])
def test_quantize_sizes_and_percentiles(k, pct):
    n = 37 if k <= 16384 else 5
    w = synthetic.random_w(n, k, seed=k)
    rng = np.random.default_rng(k)
    # heavy-tailed entries so the percentile clips something
    idx = rng.choice(n * k, size=max(1, n * k // 500), replace=False)
    w.reshape(-1)[idx] *= np.float32(10.0)
    w[0, : k // 2] = 0.0  # a row whose low ranks are all equal
    _check_quant(w, pct, "sizes")


@pytest.mark.parametrize("pct", [99.9999999, 100.0 - 1e-13, 33.333333333, 1e-6])
def test_quantize_percentile_position_edges(pct):
    w = synthetic.random_w(9, 48, seed=3)
    _check_quant(w, pct, "pct-edge")


@pytest.mark.parametrize("r", [1, 2, 3, 5, 8, 9, 12])
def test_quantize_percentile_near_top_with_duplicates(r):
    """Clip percentiles whose bound sits r ranks below the top, on rows whose
    largest magnitudes repeat (1 to 6 copies) and mix signs: the bound pair
    a[i], a[i+1] must come out the same whether it is found walking down
    from the maximum (small r) or by the radix select (larger r)."""
    k = 1024
    rng = np.random.default_rng(100 + r)
    rows = []
    for j in range(48):
        row = rng.integers(-40, 41, size=k).astype(np.float32) * np.float32(0.0005)
        top = rng.permutation(k)
        level = np.float32(0.05)
        pos = 0
        for copies in ((j % 6) + 1, (j // 6) % 4 + 1, 2, 1, 3):
            for _ in range(copies):
                row[top[pos]] = level if (pos % 2) == 0 else -level
                pos += 1
            level = np.float32(level * np.float32(0.9))
        rows.append(row)
    w = np.stack(rows)
    # pct chosen so that floor(pct / 100 * (k - 1)) = k - 1 - r, mid-way
    pct = 100.0 * ((k - 1 - r) + 0.5) / (k - 1)
    _check_quant(w, pct, "near-top r=%d" % r)


@pytest.mark.parametrize("n,k,pct", [(64, 16, 100.0), (37, 1040, 100.0), (96, 4096, 99.99),
                                      (300, 1024, 99.9), (17, 4112, 90.0), (8, 65536, 100.0)])
def test_quantize_f16_input(n, k, pct):
    """fp16 weights: the codes and scales must equal the oracle's on the
    exactly widened fp32 matrix.  The matrix mixes normal, subnormal, zero
    and large fp16 values."""
    rng = np.random.default_rng(n * 131 + k)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float16)
    w.flat[rng.integers(0, w.size, max(1, w.size // 500))] = np.float16(6.0e-6)   # subnormal
    w.flat[rng.integers(0, w.size, max(1, w.size // 500))] = np.float16(0.0)
    w.flat[rng.integers(0, w.size, max(1, w.size // 1000))] = np.float16(-3.5)
    w[0, :] = np.float16(0.0)                                                        # all-zero row
    say("quantize f16 n=%d k=%d pct=%r" % (n, k, pct))
    q_ref, s_ref, _ = oracle.quantize(w.astype(np.float32), pct)
    q, s = gpu_quantize(w, pct)
    assert np.array_equal(s, s_ref), "scales differ at rows %s" % np.nonzero(s != s_ref)[0][:5]
    assert np.array_equal(q, q_ref), "codes differ at %s" % np.argwhere(q != q_ref)[:5]


@pytest.mark.parametrize("n,k", [(64, 16), (37, 1040), (300, 1024), (96, 4096), (17, 4112), (5, 65536)])
def test_quantize_fixed_range(n, k):
    """Given per-row bounds (zero, below, at and above the absmax): codes
    and scales bit-identical to the oracle's fixed-range quantizer."""
    from gpu_util import gpu_quantize_fixed
    rng = np.random.default_rng(n + k)
    w = synthetic.random_w(n, k, n * 7 + k)
    amax = np.abs(w).max(axis=1)
    bounds = (amax * rng.choice([0.0, 0.25, 0.9, 1.0, 3.0], size=n)).astype(np.float32)
    bounds[0] = 0.0
    say("quantize fixed range n=%d k=%d" % (n, k))
    q_ref, s_ref = oracle.quantize_fixed(w, bounds)
    q, s = gpu_quantize_fixed(w, bounds)
    assert np.array_equal(s, s_ref), "scales differ at rows %s" % np.nonzero(s != s_ref)[0][:5]
    assert np.array_equal(q, q_ref), "codes differ at %s" % np.argwhere(q != q_ref)[:5]


def test_quantize_fixed_range_of_workload_bounds():
    """The outlier workload's own 99.99th-percentile bounds passed as fixed
    ranges give exactly the percentile quantizer's codes."""
    from gpu_util import gpu_quantize_fixed
    wl, x, w, q_ref, s_ref = workload_data("transformer_big_ffn_outliers_m4096_k1024_n4096")
    _, _, t = oracle.quantize(w, wl.clip_percentile)
    say("quantize fixed range of workload bounds n=%d k=%d" % (wl.n, wl.k))
    q, s = gpu_quantize_fixed(w, t)
    assert np.array_equal(s, s_ref) and np.array_equal(q, q_ref)


def test_quantize_deterministic():
    wl, x, w, q, s = workload_data("transformer_big_ffn_outliers_m4096_k1024_n4096")
    say("quantize determinism")
    a = gpu_quantize(w, wl.clip_percentile)
    b = gpu_quantize(w, wl.clip_percentile)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_empty_calls_write_nothing():
    import int8_weight_quantized_amd as qw
    torch = pytest.importorskip("torch")
    say("empty calls")
    y = torch.full((3, 5), 7, dtype=torch.int16, device="cuda:0")
    x = torch.zeros((3, 16), dtype=torch.float16, device="cuda:0")
    q = torch.zeros((5, 16), dtype=torch.int8, device="cuda:0")
    s = torch.zeros((5,), dtype=torch.float16, device="cuda:0")
    assert qw.w8a16_gemm_raw(x.data_ptr(), q.data_ptr(), s.data_ptr(), y.data_ptr(), 0, 5, 16) == 0
    assert qw.w8a16_gemm_raw(x.data_ptr(), q.data_ptr(), s.data_ptr(), y.data_ptr(), 3, 0, 16) == 0
    torch.cuda.synchronize()
    assert torch.all(y == 7)


def test_torch_binding_on_side_stream():
    import int8_weight_quantized_amd as qw
    torch = pytest.importorskip("torch")
    say("torch binding on a side stream")
    wl, x, w, q_ref, s_ref = workload_data("tiny_m1_k256_n512")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        wd = torch.from_numpy(w).to("cuda:0", non_blocking=False)
        xd = torch.from_numpy(x).to("cuda:0")
        q, s = qw.quantize_weights(wd)
        y = qw.w8a16_gemm(xd, q, s)
    stream.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint16), s_ref)
    assert_gemm_close(y.cpu().numpy(), oracle.gemm(x, q_ref, s_ref), "binding")

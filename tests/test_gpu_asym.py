"""GPU parity of the asymmetric (zero-point) quantizer and the asymmetric
W8A16 GEMM through the C ABI against the CPU oracle on the same seeded host
buffers.

  * quantizer: codes, fp16 scale bits and zero points bit-identical;
  * GEMM: max |Y - ref| <= 2e-3 * max|ref| + 1e-3 on every kernel path,
    bit-exact where the arithmetic is exact in fp32, and bit-identical to
    the symmetric GEMM when every zero point is 0.
"""

import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import assert_gemm_close, gpu_gemm, say, torch_mod, dev, host

pytestmark = pytest.mark.gpu

GEMV, MFMA, SKINNY = 1, 2, 3


def gpu_quantize_asym(w):
    import int8_weight_quantized_amd as qw
    torch = torch_mod()
    n, k = w.shape
    wd = dev(np.ascontiguousarray(w, dtype=np.float32))
    qd = torch.full((n, k), 99, dtype=torch.int8, device="cuda:0")
    sd = torch.full((n,), 0x5555, dtype=torch.int16, device="cuda:0")
    zd = torch.full((n,), 77, dtype=torch.int8, device="cuda:0")
    st = qw.quantize_weights_asym_raw(wd.data_ptr(), n, k, qd.data_ptr(), sd.data_ptr(), zd.data_ptr(),
                                      int(torch.cuda.current_stream().cuda_stream))
    assert st == 0, qw.status_string(st)
    return host(qd), host(sd).view(np.uint16), host(zd)


def gpu_gemm_asym(x, q, s_bits, z, path=0):
    import int8_weight_quantized_amd as qw
    torch = torch_mod()
    m, k = x.shape
    n = q.shape[0]
    xd = dev(np.ascontiguousarray(x, dtype=np.float16).view(np.int16))
    qd = dev(np.ascontiguousarray(q, dtype=np.int8))
    sd = dev(np.ascontiguousarray(s_bits, dtype=np.uint16).view(np.int16))
    zd = dev(np.ascontiguousarray(z, dtype=np.int8))
    yd = torch.full((m, n), 0x7e00, dtype=torch.int16, device="cuda:0")  # NaN canary
    st = qw.w8a16_gemm_asym_raw(xd.data_ptr(), qd.data_ptr(), sd.data_ptr(), zd.data_ptr(), yd.data_ptr(),
                                m, n, k, int(torch.cuda.current_stream().cuda_stream), path)
    assert st == 0, qw.status_string(st)
    return host(yd).view(np.float16)


def _weights(n, k, seed):
    """Rows of every kind: mixed sign, all positive, all negative, offset
    away from zero, all zero, and a constant row."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[1::6] = np.abs(w[1::6])
    w[2::6] = -np.abs(w[2::6])
    w[3::6] = w[3::6] + np.float32(0.1)
    w[4::6] = 0.0
    w[5::6] = np.float32(-0.37)
    return w


@pytest.mark.parametrize("n,k", [(64, 16), (37, 1040), (300, 1024), (96, 4096), (17, 4112), (6, 65536)])
def test_quantize_asym(n, k):
    w = _weights(n, k, n * 13 + k)
    say("quantize asym n=%d k=%d" % (n, k))
    q_ref, s_ref, z_ref = oracle.quantize_asym(w)
    q, s, z = gpu_quantize_asym(w)
    assert np.array_equal(s, s_ref), "scales differ at rows %s" % np.nonzero(s != s_ref)[0][:5]
    assert np.array_equal(z, z_ref), "zero points differ at rows %s" % np.nonzero(z != z_ref)[0][:5]
    assert np.array_equal(q, q_ref), "codes differ at %s" % np.argwhere(q != q_ref)[:5]


def test_quantize_asym_outlier_workload():
    wl = synthetic.BY_NAME["transformer_big_ffn_outliers_m4096_k1024_n4096"]
    _, w = synthetic.make_inputs(wl)
    say("quantize asym %s" % wl.name)
    q_ref, s_ref, z_ref = oracle.quantize_asym(w)
    q, s, z = gpu_quantize_asym(w)
    assert np.array_equal(s, s_ref) and np.array_equal(z, z_ref) and np.array_equal(q, q_ref)


SHAPES = [(1, 1000, 272), (2, 300, 2064), (4, 64, 16), (8, 517, 2064), (17, 300, 528), (65, 130, 96),
          (130, 260, 4112), (300, 513, 1040), (24, 517, 2064), (20, 25000, 2064)]


@pytest.mark.parametrize("m,n,k", SHAPES)
def test_gemm_asym_every_path(m, n, k):
    x = synthetic.random_x(m, k, m + n)
    w = _weights(n, k, m * 3 + n)
    q, s, z = oracle.quantize_asym(w)
    ref = oracle.gemm_asym(x, q, s, z)
    for path in (0, GEMV, SKINNY, MFMA):
        if path == GEMV and m > 8:
            continue
        say("gemm asym path=%d m=%d n=%d k=%d" % (path, m, n, k))
        assert_gemm_close(gpu_gemm_asym(x, q, s, z, path), ref, "asym path %d %dx%dx%d" % (path, m, n, k))


@pytest.mark.parametrize("path", [GEMV, SKINNY, MFMA])
@pytest.mark.parametrize("m,n,k", [(1, 96, 512), (4, 200, 1024), (8, 130, 2048)])
def test_gemm_asym_exact_arithmetic_bitexact(path, m, n, k):
    """X in {-1,0,1}, power-of-two scales, any zero points: q - z is exact in
    fp16 and every partial sum is exact in fp32 (k * 255 < 2^24), so Y is the
    fp16 rounding of the exact value, bit for bit."""
    rng = np.random.default_rng(m + n + k + path)
    x = rng.integers(-1, 2, size=(m, k)).astype(np.float16)
    q = rng.integers(-128, 128, size=(n, k)).astype(np.int8)
    z = rng.integers(-128, 128, size=n).astype(np.int8)
    s = (2.0 ** (-rng.integers(0, 11, size=n))).astype(np.float16).view(np.uint16)
    say("gemm asym exact path=%d m=%d n=%d k=%d" % (path, m, n, k))
    y = gpu_gemm_asym(x, q, s, z, path)
    want = oracle.f64_to_f16_bits(oracle.gemm_asym(x, q, s, z))
    assert np.array_equal(y.view(np.uint16), want)


@pytest.mark.parametrize("m,n,k", [(1, 1000, 272), (8, 517, 2064), (300, 513, 1040)])
def test_gemm_asym_zero_points_zero_is_symmetric(m, n, k):
    """With every zero point 0 the asymmetric call runs the same arithmetic
    as the symmetric one: outputs bit-identical on every path."""
    x = synthetic.random_x(m, k, 5 * m + n)
    w = synthetic.random_w(n, k, m + 7)
    q, s, _ = oracle.quantize(w, 100.0)
    z = np.zeros(n, dtype=np.int8)
    for path in (GEMV, SKINNY, MFMA):
        if path == GEMV and m > 8:
            continue
        say("gemm asym z=0 path=%d m=%d n=%d k=%d" % (path, m, n, k))
        a = gpu_gemm_asym(x, q, s, z, path)
        b = gpu_gemm(x, q, s, path=path)
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("name", ["chatglm2_decode_m1_k4096_n27392", "transformer_big_ffn_outliers_m4096_k1024_n4096"])
def test_gemm_asym_workload(name):
    wl = synthetic.BY_NAME[name]
    x, w = synthetic.make_inputs(wl)
    say("quantize asym + gemm asym %s" % name)
    q, s, z = gpu_quantize_asym(w)
    q_ref, s_ref, z_ref = oracle.quantize_asym(w)
    assert np.array_equal(q, q_ref) and np.array_equal(s, s_ref) and np.array_equal(z, z_ref)
    y = gpu_gemm_asym(x, q, s, z)
    rng = np.random.default_rng(99)
    mr = np.unique(np.r_[0, wl.m - 1, rng.integers(0, wl.m, 4)])
    mi = np.concatenate([np.repeat(mr, wl.n), rng.integers(0, wl.m, 4096)])
    ni = np.concatenate([np.tile(np.arange(wl.n), len(mr)), rng.integers(0, wl.n, 4096)])
    assert_gemm_close(y[mi, ni], oracle.gemm_asym_sampled(x, q, s, z, mi, ni), name + " asym (sampled)")
    assert np.all(np.isfinite(y.astype(np.float32)))

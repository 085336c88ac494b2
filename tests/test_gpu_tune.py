"""Per-shape autotuning of the W8A16 kernel choice on the GPU: the tuning
call's result and every later automatic call for the same shape bucket
match the oracle, and the record steers the automatic choice."""

import numpy as np
import pytest

import oracle
import synthetic
from gpu_util import assert_gemm_close, dev, host, say, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def clean_records():
    import int8_weight_quantized_amd as qw
    qw.tune_reset()
    yield
    qw.tune_reset()


def _tune(x, q, s):
    import int8_weight_quantized_amd as qw
    torch = torch_mod()
    m, k = x.shape
    n = q.shape[0]
    xd = dev(np.ascontiguousarray(x, dtype=np.float16).view(np.int16))
    qd = dev(q)
    sd = dev(np.ascontiguousarray(s, dtype=np.uint16).view(np.int16))
    yd = torch.full((m, n), 0x7e00, dtype=torch.int16, device="cuda:0")
    st = qw.w8a16_gemm_tune_raw(xd.data_ptr(), qd.data_ptr(), sd.data_ptr(), yd.data_ptr(), m, n, k,
                                int(torch.cuda.current_stream().cuda_stream))
    assert st == 0, qw.status_string(st)
    return host(yd).view(np.float16)


@pytest.mark.parametrize("m,n,k", [(3, 27392, 1024), (8, 4608, 4096), (40, 4608, 1040), (512, 4096, 1024),
                                   (130, 9000, 272)])
def test_tune_records_and_steers(m, n, k):
    import int8_weight_quantized_amd as qw
    from gpu_util import gpu_gemm
    x = synthetic.random_x(m, k, m + n)
    w = synthetic.random_w(n, k, m + 1)
    q, s, _ = oracle.quantize(w, 100.0)
    ref = oracle.gemm(x, q, s)
    assert qw.tuned_choice(m, n, k) is None
    say("gemm tune m=%d n=%d k=%d" % (m, n, k))
    y_tune = _tune(x, q, s)
    assert_gemm_close(y_tune, ref, "tune %dx%dx%d" % (m, n, k))
    choice = qw.tuned_choice(m, n, k)
    assert choice is not None
    path, tile = choice
    assert path in ("gemv", "skinny", "mfma") and (tile is None) == (path != "mfma")
    say("tuned choice %s %s" % (path, tile))
    assert qw.auto_path(m, n, k) == path
    if path == "mfma":
        assert qw.mfma_tile(m, n, k) == tile
    y_auto = gpu_gemm(x, q, s)
    assert np.array_equal(y_auto.view(np.uint16), y_tune.view(np.uint16)), "auto call must run the tuned kernel"
    # same bucket (m rounded up to a multiple of 8) shares the record
    m2 = (m + 7) // 8 * 8
    assert qw.tuned_choice(m2, n, k) == choice
    assert qw.tuned_choice(m2 + 1, n, k) is None
    qw.tune_reset()
    assert qw.tuned_choice(m, n, k) is None


def _tune_w8a8(qx, sx, q, s):
    import int8_weight_quantized_amd as qw
    torch = torch_mod()
    m, k = qx.shape
    n = q.shape[0]
    qxd, sxd = dev(np.ascontiguousarray(qx, dtype=np.int8)), dev(np.ascontiguousarray(sx, dtype=np.uint16).view(np.int16))
    qd, sd = dev(np.ascontiguousarray(q, dtype=np.int8)), dev(np.ascontiguousarray(s, dtype=np.uint16).view(np.int16))
    yd = torch.full((m, n), 0x7e00, dtype=torch.int16, device="cuda:0")
    st = qw.w8a8_gemm_tune_raw(qxd.data_ptr(), sxd.data_ptr(), qd.data_ptr(), sd.data_ptr(), yd.data_ptr(), m, n, k,
                               int(torch.cuda.current_stream().cuda_stream))
    assert st == 0, qw.status_string(st)
    return host(yd).view(np.float16)


@pytest.mark.parametrize("m,n,k", [(8, 4608, 4096), (96, 4608, 1040), (300, 4096, 1024), (129, 600, 528)])
def test_w8a8_tune_records_and_steers(m, n, k):
    """The W8A8 records: the tuning call's result matches the oracle, the
    record steers qw_w8a8_gemm (bit-identical output), its bucket is shared,
    and it is kept apart from the W8A16 records."""
    import int8_weight_quantized_amd as qw
    from gpu_util import assert_w8a8_close, gpu_w8a8
    x = synthetic.random_x(m, k, m + n)
    w = synthetic.random_w(n, k, m + 1)
    qx, sx, _ = oracle.quantize(x.astype(np.float32), 100.0)
    q, s, _ = oracle.quantize(w, 100.0)
    ref = oracle.w8a8_gemm(qx, sx, q, s)
    assert qw.w8a8_tuned_choice(m, n, k) is None
    say("w8a8 gemm tune m=%d n=%d k=%d" % (m, n, k))
    y_tune = _tune_w8a8(qx, sx, q, s)
    assert_w8a8_close(y_tune, ref, "w8a8 tune %dx%dx%d" % (m, n, k))
    choice = qw.w8a8_tuned_choice(m, n, k)
    assert choice is not None and qw.tuned_choice(m, n, k) is None
    path, tile = choice
    assert path in ("skinny", "mfma") and (tile is None) == (path == "skinny")
    assert tile in (None, (256, 128), (256, 64), (128, 64))
    say("w8a8 tuned choice %s %s" % (path, tile))
    assert qw.w8a8_auto_path(m, n, k) == path
    if path == "mfma":
        assert qw.w8a8_tile(m, n, k) == tile
    y_auto = gpu_w8a8(qx, sx, q, s)
    assert np.array_equal(y_auto.view(np.uint16), y_tune.view(np.uint16)), "auto call must run the tuned kernel"
    m2 = (m + 7) // 8 * 8
    assert qw.w8a8_tuned_choice(m2, n, k) == choice
    qw.tune_reset()
    assert qw.w8a8_tuned_choice(m, n, k) is None

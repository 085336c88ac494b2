"""The Python binding's argument checks, without a GPU.

The C ABI sees raw pointers only, so the binding is what keeps a wrong
device, dtype, shape or layout from reaching a kernel (a host pointer or an
undersized output would become an out-of-bounds access on the GPU).  Each
call validates its arguments in a helper that runs before any launch; these
tests drive every rejection of those helpers with meta-device tensors (the
first operand's device is the one every other tensor must share) and check
that the public calls refuse CPU tensors before reaching the library."""

import pytest

torch = pytest.importorskip("torch")
qw = pytest.importorskip("int8_weight_quantized_amd")

META = torch.device("meta")


def t(shape, dtype, device=META):
    return torch.empty(shape, dtype=dtype, device=device)


M, N, K = 3, 32, 64


def gemm_operands():
    return (t((M, K), torch.float16), t((N, K), torch.int8), t((N,), torch.float16))


def test_valid_arguments_pass():
    x, q, s = gemm_operands()
    m, n, k, cap, y = qw._validate_gemm(x, q, s, None, "auto", META)
    assert (m, n, k, cap) == (M, N, K, 0) and tuple(y.shape) == (M, N) and y.dtype == torch.float16
    m, n, k, cap, y = qw._validate_gemm(x, q, s, t((M, N), torch.float16), "mfma", META,
                                        ol=(t((N, 2), torch.int32), t((N, 2), torch.float32)),
                                        zeros=t((N,), torch.int8))
    assert cap == 2
    f16, n, k, qo, so = qw._validate_quantize(t((N, K), torch.float32), None, META)
    assert not f16 and (n, k) == (N, K) and tuple(qo.shape) == (N, K) and tuple(so.shape) == (N,)
    f16, *_ = qw._validate_quantize(t((N, K), torch.float16), (t((N, K), torch.int8), t((N,), torch.float16)), META)
    assert f16


@pytest.mark.parametrize("case", [
    "x_dtype", "x_ndim", "x_noncontig", "x_other_device", "q_dtype", "q_k_mismatch", "q_noncontig",
    "q_other_device", "scales_len", "scales_dtype", "scales_other_device", "out_shape", "out_dtype",
    "out_noncontig", "out_other_device", "out_not_tensor", "path",
])
def test_gemm_rejections(case):
    x, q, s = gemm_operands()
    out, path = None, "auto"
    cpu = torch.device("cpu")
    if case == "x_dtype":
        x = t((M, K), torch.float32)
    elif case == "x_ndim":
        x = t((M * K,), torch.float16)
    elif case == "x_noncontig":
        x = t((K, M), torch.float16).t()
    elif case == "x_other_device":
        x = t((M, K), torch.float16, cpu)
    elif case == "q_dtype":
        q = t((N, K), torch.uint8)
    elif case == "q_k_mismatch":
        q = t((N, K + 16), torch.int8)
    elif case == "q_noncontig":
        q = t((K, N), torch.int8).t()
    elif case == "q_other_device":
        q = t((N, K), torch.int8, cpu)
    elif case == "scales_len":
        s = t((N + 1,), torch.float16)
    elif case == "scales_dtype":
        s = t((N,), torch.float32)
    elif case == "scales_other_device":
        s = t((N,), torch.float16, cpu)
    elif case == "out_shape":
        out = t((M, N - 1), torch.float16)
    elif case == "out_dtype":
        out = t((M, N), torch.float32)
    elif case == "out_noncontig":
        out = t((N, M), torch.float16).t()
    elif case == "out_other_device":
        out = t((M, N), torch.float16, cpu)
    elif case == "out_not_tensor":
        out = [1, 2]
    elif case == "path":
        path = "fastest"
    with pytest.raises((TypeError, ValueError)):
        qw._validate_gemm(x, q, s, out, path, META)


@pytest.mark.parametrize("case", ["idx_dtype", "val_dtype", "idx_rows", "val_cols", "idx_noncontig",
                                  "val_other_device"])
def test_side_list_rejections(case):
    x, q, s = gemm_operands()
    idx, val = t((N, 2), torch.int32), t((N, 2), torch.float32)
    if case == "idx_dtype":
        idx = t((N, 2), torch.int64)
    elif case == "val_dtype":
        val = t((N, 2), torch.float16)
    elif case == "idx_rows":
        idx = t((N - 1, 2), torch.int32)
    elif case == "val_cols":
        val = t((N, 3), torch.float32)
    elif case == "idx_noncontig":
        idx = t((2, N), torch.int32).t()
    elif case == "val_other_device":
        val = t((N, 2), torch.float32, torch.device("cpu"))
    with pytest.raises((TypeError, ValueError)):
        qw._validate_gemm(x, q, s, None, "auto", META, ol=(idx, val))


@pytest.mark.parametrize("case", ["zeros_len", "zeros_dtype", "zeros_other_device"])
def test_zero_point_rejections(case):
    x, q, s = gemm_operands()
    z = {"zeros_len": t((N - 1,), torch.int8), "zeros_dtype": t((N,), torch.uint8),
         "zeros_other_device": t((N,), torch.int8, torch.device("cpu"))}[case]
    with pytest.raises((TypeError, ValueError)):
        qw._validate_gemm(x, q, s, None, "auto", META, zeros=z)


@pytest.mark.parametrize("case", ["qx_dtype", "sx_len", "sx_dtype", "sx_other_device"])
def test_w8a8_rejections(case):
    qx, q, s, sx = t((M, K), torch.int8), t((N, K), torch.int8), t((N,), torch.float16), t((M,), torch.float16)
    if case == "qx_dtype":
        qx = t((M, K), torch.float16)
    elif case == "sx_len":
        sx = t((M + 1,), torch.float16)
    elif case == "sx_dtype":
        sx = t((M,), torch.float32)
    elif case == "sx_other_device":
        sx = t((M,), torch.float16, torch.device("cpu"))
    with pytest.raises((TypeError, ValueError)):
        qw._validate_gemm(qx, q, s, None, None, META, a8=True, sx=sx)


@pytest.mark.parametrize("out", [
    "one_tensor", "q_shape", "q_dtype", "scales_shape", "scales_dtype", "q_other_device", "three",
])
def test_quantize_output_rejections(out):
    w = t((N, K), torch.float32)
    q, s = t((N, K), torch.int8), t((N,), torch.float16)
    outs = {"one_tensor": q, "q_shape": (t((N, K - 16), torch.int8), s), "q_dtype": (t((N, K), torch.uint8), s),
            "scales_shape": (q, t((N - 1,), torch.float16)), "scales_dtype": (q, t((N,), torch.float32)),
            "q_other_device": (t((N, K), torch.int8, torch.device("cpu")), s), "three": (q, s, s)}[out]
    with pytest.raises((TypeError, ValueError)):
        qw._validate_quantize(w, outs, META)


def test_quantize_input_rejections():
    with pytest.raises(TypeError):
        qw._validate_quantize(t((N, K), torch.float64), None, META)
    with pytest.raises(ValueError):
        qw._validate_quantize(t((N * K,), torch.float32), None, META)
    with pytest.raises(ValueError):
        qw._validate_quantize(t((K, N), torch.float32).t(), None, META)


def test_fixed_range_rejections():
    w = t((N, K), torch.float32)
    for bounds, out in ((t((N + 1,), torch.float32), None), (t((N,), torch.float16), None),
                        (t((N,), torch.float32, torch.device("cpu")), None),
                        (t((N,), torch.float32), (t((N, K), torch.int8), t((N + 2,), torch.float16)))):
        with pytest.raises((TypeError, ValueError)):
            qw._validate_fixed_range(w, bounds, out, META)
    n, k, q, s = qw._validate_fixed_range(w, t((N,), torch.float32), None, META)
    assert (n, k) == (N, K)


def test_public_calls_refuse_cpu_tensors_before_the_library():
    cpu = torch.device("cpu")
    x, q, s = (t((M, K), torch.float16, cpu), t((N, K), torch.int8, cpu), t((N,), torch.float16, cpu))
    w = t((N, K), torch.float32, cpu)
    calls = [
        lambda: qw.quantize_weights(w),
        lambda: qw.quantize_weights_fixed_range(w, t((N,), torch.float32, cpu)),
        lambda: qw.quantize_weights_outliers(w, 99.0),
        lambda: qw.quantize_weights_asym(w),
        lambda: qw.w8a16_gemm(x, q, s),
        lambda: qw.w8a16_gemm_tune(x, q, s),
        lambda: qw.w8a16_gemm_asym(x, q, s, t((N,), torch.int8, cpu)),
        lambda: qw.w8a16_gemm_outliers(x, q, s, t((N, 1), torch.int32, cpu), t((N, 1), torch.float32, cpu)),
        lambda: qw.w8a8_gemm(t((M, K), torch.int8, cpu), t((M,), torch.float16, cpu), q, s),
        lambda: qw.quantize_activations(x),
        lambda: qw.w8a16_gemm_tile(x, q, s, (256, 256)),
        lambda: qw.w8a8_gemm_tile(t((M, K), torch.int8, cpu), t((M,), torch.float16, cpu), q, s, (256, 256)),
    ]
    for call in calls:
        with pytest.raises(ValueError, match="GPU"):
            call()


def test_gemm_tile_argument_rejections():
    """A tile outside the built set, or zero points together with side
    lists, is refused before any tensor is looked at."""
    x, q, s = gemm_operands()
    for tile in ((256, 512), (64, 64), (256,), "256256"):
        with pytest.raises(ValueError, match="tile"):
            qw.w8a16_gemm_tile(x, q, s, tile)
    with pytest.raises(ValueError, match="zeros or outliers"):
        qw.w8a16_gemm_tile(x, q, s, (256, 256), zeros=t((N,), torch.int8),
                           outliers=(t((N, 1), torch.int32), t((N, 1), torch.float32)))
    assert set(qw.MFMA_TILES) == {(256, 256), (256, 128), (256, 64), (128, 128), (128, 64)}
    qx = t((M, K), torch.int8)
    for tile in ((128, 128), (512, 256)):
        with pytest.raises(ValueError, match="tile"):
            qw.w8a8_gemm_tile(qx, t((M,), torch.float16), q, s, tile)

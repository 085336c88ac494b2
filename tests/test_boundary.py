"""The C-ABI boundary on the CPU: the library loads, exports every symbol the
header declares, and rejects every invalid call with the documented status
before touching the GPU (no compute call is made here)."""

import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qw.h")

qw = pytest.importorskip("int8_weight_quantized_amd")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"QW_API\s+[\w\s\*]+?\b(qw_\w+)\s*\(", text)))


def _exported_symbols():
    out = subprocess.run(["nm", "-D", "--defined-only", qw.LIBRARY_PATH], capture_output=True,
                         text=True, check=True).stdout
    return {line.split()[-1] for line in out.splitlines() if line.strip()}


def test_header_declares_the_entry_points():
    decl = _declared_functions()
    for name in ("qw_quantize_weights", "qw_quantize_weights_f16", "qw_w8a16_gemm", "qw_w8a16_gemm_path",
                 "qw_w8a16_gemm_auto_path", "qw_w8a16_gemm_mfma_tile", "qw_w8a8_gemm",
                 "qw_w8a8_gemm_mfma_tile", "qw_w8a8_gemm_auto_path", "qw_quantize_weights_fixed_range",
                 "qw_quantize_weights_asym",
                 "qw_w8a16_gemm_asym", "qw_w8a16_gemm_asym_path", "qw_outlier_capacity",
                 "qw_quantize_weights_outliers", "qw_w8a16_gemm_outliers", "qw_w8a16_gemm_outliers_path",
                 "qw_w8a16_gemm_tune", "qw_w8a16_gemm_tuned_choice", "qw_w8a16_gemm_tune_reset",
                 "qw_w8a8_gemm_tune", "qw_w8a8_gemm_tuned_choice",
                 "qw_status_string", "qw_version"):
        assert name in decl


def test_library_exports_every_declared_symbol():
    exported = _exported_symbols()
    missing = [f for f in _declared_functions() if f not in exported]
    assert not missing, missing
    lib = qw.library()
    for f in _declared_functions():
        assert hasattr(lib, f)


def test_library_is_independent_of_the_oracle():
    exported = _exported_symbols()
    assert not any(s.startswith("oracle_") for s in exported)
    deps = subprocess.run(["ldd", qw.LIBRARY_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in deps


def test_one_hip_runtime_whichever_loads_first():
    """Loading libqw.so before torch must not map a second HIP runtime (torch
    would then see no GPU and its stream handles would be foreign to libqw)."""
    pytest.importorskip("torch")
    code = (
        "import int8_weight_quantized_amd as qw; qw.library(); import torch\n"
        "paths = set(l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l)\n"
        "print(len(paths)); print(sorted(paths))\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.splitlines()[0] == "1", out.stdout


def test_status_strings_and_version():
    assert qw.version() >= 100
    for st in range(5):
        assert qw.status_string(st)
    assert qw.status_string(99) == "unknown status"


# Fake, never-dereferenced addresses: every call below must be rejected on the
# host before anything is enqueued.
A = 1 << 20      # 16-byte aligned
B = 2 << 20
C = 3 << 20
D = 4 << 20
E = 5 << 20


@pytest.mark.parametrize("args,status", [
    ((A, -1, 16, 100.0, B, C), qw.QW_ERROR_INVALID_VALUE),          # n < 0
    ((A, 4, 0, 100.0, B, C), qw.QW_ERROR_INVALID_VALUE),            # k == 0
    ((A, 4, -16, 100.0, B, C), qw.QW_ERROR_INVALID_VALUE),          # k < 0
    ((A, 4, 16, 0.0, B, C), qw.QW_ERROR_INVALID_VALUE),             # pct == 0
    ((A, 4, 16, 100.0001, B, C), qw.QW_ERROR_INVALID_VALUE),        # pct > 100
    ((A, 4, 16, float("nan"), B, C), qw.QW_ERROR_INVALID_VALUE),    # pct NaN
    ((0, 4, 16, 100.0, B, C), qw.QW_ERROR_INVALID_VALUE),           # null w
    ((A, 4, 16, 100.0, 0, C), qw.QW_ERROR_INVALID_VALUE),           # null q
    ((A, 4, 16, 100.0, B, 0), qw.QW_ERROR_INVALID_VALUE),           # null scales
    ((A, 4, 24, 100.0, B, C), qw.QW_ERROR_UNSUPPORTED),             # k % 16
    ((A, 4, 65536 + 16, 100.0, B, C), qw.QW_ERROR_UNSUPPORTED),     # k too large
    ((A, 1 << 31, 16, 100.0, B, C), qw.QW_ERROR_UNSUPPORTED),       # n too large
    ((A + 4, 4, 16, 100.0, B, C), qw.QW_ERROR_MISALIGNED),
    ((A, 4, 16, 100.0, B + 8, C), qw.QW_ERROR_MISALIGNED),
    ((A, 4, 16, 100.0, B, C + 2), qw.QW_ERROR_MISALIGNED),
    ((A, 4, 16, 100.0, A + 64, C), qw.QW_ERROR_INVALID_VALUE),      # q overlaps w
    ((A, 4, 16, 100.0, B, A + 16), qw.QW_ERROR_INVALID_VALUE),      # scales overlap w
    ((A, 4, 16, 100.0, B, B + 32), qw.QW_ERROR_INVALID_VALUE),      # scales overlap q
])
def test_quantize_rejects(args, status):
    assert qw.quantize_weights_raw(*args) == status


@pytest.mark.parametrize("args,status", [
    ((A, -1, 16, 100.0, B, C), qw.QW_ERROR_INVALID_VALUE),          # n < 0
    ((A, 4, 16, 0.0, B, C), qw.QW_ERROR_INVALID_VALUE),             # pct == 0
    ((0, 4, 16, 100.0, B, C), qw.QW_ERROR_INVALID_VALUE),           # null w
    ((A, 4, 24, 100.0, B, C), qw.QW_ERROR_UNSUPPORTED),             # k % 16
    ((A + 8, 4, 16, 100.0, B, C), qw.QW_ERROR_MISALIGNED),
    ((A, 4, 16, 100.0, A + 96, C), qw.QW_ERROR_INVALID_VALUE),      # q inside w (4 x 16 fp16 = 128 bytes)
    ((A, 4, 16, 100.0, B, A + 112), qw.QW_ERROR_INVALID_VALUE),     # scales inside w's last row
])
def test_quantize_f16_rejects(args, status):
    assert qw.quantize_weights_f16_raw(*args) == status


@pytest.mark.parametrize("args,status", [
    ((A, -1, 16, D, B, C), qw.QW_ERROR_INVALID_VALUE),              # n < 0
    ((A, 4, 0, D, B, C), qw.QW_ERROR_INVALID_VALUE),                # k == 0
    ((A, 4, 16, 0, B, C), qw.QW_ERROR_INVALID_VALUE),               # null bounds
    ((0, 4, 16, D, B, C), qw.QW_ERROR_INVALID_VALUE),               # null w
    ((A, 4, 24, D, B, C), qw.QW_ERROR_UNSUPPORTED),                 # k % 16
    ((A, 4, 16, D + 4, B, C), qw.QW_ERROR_MISALIGNED),              # bounds
    ((A, 4, 16, D, B, D), qw.QW_ERROR_INVALID_VALUE),               # scales overlap bounds
    ((A, 4, 16, D, D, C), qw.QW_ERROR_INVALID_VALUE),               # q overlaps bounds
    ((A, 4, 16, D, A + 128, C), qw.QW_ERROR_INVALID_VALUE),         # q inside w (4 x 16 fp32)
])
def test_quantize_fixed_range_rejects(args, status):
    assert qw.quantize_weights_fixed_range_raw(*args) == status


@pytest.mark.parametrize("args,status", [
    ((A, -1, 16, B, C, D), qw.QW_ERROR_INVALID_VALUE),              # n < 0
    ((A, 4, 0, B, C, D), qw.QW_ERROR_INVALID_VALUE),                # k == 0
    ((A, 4, 16, B, C, 0), qw.QW_ERROR_INVALID_VALUE),               # null zeros
    ((A, 4, 24, B, C, D), qw.QW_ERROR_UNSUPPORTED),                 # k % 16
    ((A, 4, 16, B, C, D + 1), qw.QW_ERROR_MISALIGNED),              # zeros
    ((A, 4, 16, B, C, C), qw.QW_ERROR_INVALID_VALUE),               # zeros overlap scales
    ((A, 4, 16, B, C, B + 16), qw.QW_ERROR_INVALID_VALUE),          # zeros overlap q
    ((A, 4, 16, B, C, A + 240), qw.QW_ERROR_INVALID_VALUE),         # zeros inside w
])
def test_quantize_asym_rejects(args, status):
    assert qw.quantize_weights_asym_raw(*args) == status


@pytest.mark.parametrize("args,status", [
    ((A, B, C, 0, D, 1, 4, 16), qw.QW_ERROR_INVALID_VALUE),         # null zeros
    ((A, B, C, E + 1, D, 1, 4, 16), qw.QW_ERROR_MISALIGNED),        # zeros
    ((A, B, C, D, D, 1, 4, 16), qw.QW_ERROR_INVALID_VALUE),         # y overlaps zeros
    ((A, B, C, E, D, 1, 4, 24), qw.QW_ERROR_UNSUPPORTED),           # k % 16
    ((A, B, C, E, D, -1, 4, 16), qw.QW_ERROR_INVALID_VALUE),
])
def test_gemm_asym_rejects(args, status):
    assert qw.w8a16_gemm_asym_raw(*args) == status


def test_outlier_capacity_matches_oracle():
    import oracle
    for k in (16, 48, 64, 1024, 1040, 4096, 4112, 65536):
        for pct in (100.0, 99.9999, 99.99, 99.9, 99.0, 95.0, 90.0, 50.0, 1e-6):
            assert qw.outlier_capacity(k, pct) == oracle.outlier_capacity(k, pct), (k, pct)
    with pytest.raises(ValueError):
        qw.outlier_capacity(16, 0.0)


F = 6 << 20


@pytest.mark.parametrize("args,status", [
    ((A, 4, 1024, 99.99, B, C, D, E, 0), qw.QW_ERROR_INVALID_VALUE),      # cap below capacity (1)
    ((A, 4, 16, 99.99, B, C, D, E, 17), qw.QW_ERROR_INVALID_VALUE),       # cap above k
    ((A, 4, 16, 90.0, B, C, 0, E, 2), qw.QW_ERROR_INVALID_VALUE),         # null idx
    ((A, 4, 16, 90.0, B, C, D, 0, 2), qw.QW_ERROR_INVALID_VALUE),         # null val
    ((A, 4, 16, 90.0, B, C, D + 4, E, 2), qw.QW_ERROR_MISALIGNED),
    ((A, 4, 16, 90.0, B, C, D, E + 8, 2), qw.QW_ERROR_MISALIGNED),
    ((A, 4, 16, 90.0, B, C, D, D + 16, 2), qw.QW_ERROR_INVALID_VALUE),    # val overlaps idx (4 x 2 x 4 B)
    ((A, 4, 16, 90.0, B, C, A + 32, E, 2), qw.QW_ERROR_INVALID_VALUE),    # idx inside w
    ((A, 4, 16, 90.0, B, C, D, C, 2), qw.QW_ERROR_INVALID_VALUE),         # val overlaps scales
    ((A, 4, 16, 0.0, B, C, D, E, 2), qw.QW_ERROR_INVALID_VALUE),          # bad percentile
])
def test_quantize_outliers_rejects(args, status):
    assert qw.quantize_weights_outliers_raw(*args) == status


@pytest.mark.parametrize("args,status", [
    ((A, B, C, D, E, -1, F, 1, 4, 16), qw.QW_ERROR_INVALID_VALUE),       # cap < 0
    ((A, B, C, D, E, 17, F, 1, 4, 16), qw.QW_ERROR_INVALID_VALUE),       # cap > k
    ((A, B, C, 0, E, 2, F, 1, 4, 16), qw.QW_ERROR_INVALID_VALUE),        # null idx
    ((A, B, C, D + 4, E, 2, F, 1, 4, 16), qw.QW_ERROR_MISALIGNED),
    ((A, B, C, D, E, 2, D, 1, 4, 16), qw.QW_ERROR_INVALID_VALUE),        # y overlaps idx
    ((A, B, C, D, E, 2, F, 1, 4, 24), qw.QW_ERROR_UNSUPPORTED),          # k % 16
])
def test_gemm_outliers_rejects(args, status):
    assert qw.w8a16_gemm_outliers_raw(*args) == status


def test_gemm_outliers_mfma_slot_limit():
    # the MFMA kernel stages at most 4 slots per row; forcing it with more
    # is refused before anything is launched
    assert qw.w8a16_gemm_outliers_raw(A, B, C, D, E, 5, F, 64, 64, 64, 0, 2) == qw.QW_ERROR_UNSUPPORTED


@pytest.mark.parametrize("args,status", [
    ((A, B, C, 0, 0, 0, 0, D, 4, 4, 16, 256000), qw.QW_ERROR_INVALID_VALUE),        # no such tile
    ((A, B, C, 0, 0, 0, 0, D, 4, 4, 16, 0), qw.QW_ERROR_INVALID_VALUE),             # tile 0
    ((A, B, C, E, A, B, 2, D, 4, 4, 16, 256256), qw.QW_ERROR_INVALID_VALUE),        # zeros and side lists
    ((A, B, C, 0, 0, B, 2, D, 4, 4, 16, 256256), qw.QW_ERROR_INVALID_VALUE),        # cap > 0, null idx
    ((A, B, C, 0, 0, 0, -1, D, 4, 4, 16, 256256), qw.QW_ERROR_INVALID_VALUE),       # cap < 0
    ((A, B, C, 0, 0, 0, 0, D, -1, 4, 16, 256256), qw.QW_ERROR_INVALID_VALUE),       # m < 0
    ((0, B, C, 0, 0, 0, 0, D, 4, 4, 16, 256256), qw.QW_ERROR_INVALID_VALUE),        # null x
    ((A, B, C, 0, 0, 0, 0, D, 4, 4, 24, 256256), qw.QW_ERROR_UNSUPPORTED),          # k % 16
    ((A, B, C, 0, 0, 0, 0, D, 4, 4, qw.PINGPONG_MAX_K + 16, 256256), qw.QW_ERROR_UNSUPPORTED),  # k limit
    ((A, B, C, 0, E, F, 5, D, 4, 4, 64, 256128), qw.QW_ERROR_UNSUPPORTED),          # > 4 slots on MFMA
    ((A + 8, B, C, 0, 0, 0, 0, D, 4, 4, 16, 128064), qw.QW_ERROR_MISALIGNED),       # misaligned x
])
def test_gemm_tile_rejects(args, status):
    assert qw.w8a16_gemm_tile_raw(*args) == status


@pytest.mark.parametrize("args,status", [
    ((A, B, C, D, E, 4, 4, 16, 128128), qw.QW_ERROR_INVALID_VALUE),     # not a W8A8 tile
    ((A, B, C, D, E, 4, 4, 16, 0), qw.QW_ERROR_INVALID_VALUE),          # tile 0
    ((A, B, C, D, E, -1, 4, 16, 256256), qw.QW_ERROR_INVALID_VALUE),    # m < 0
    ((0, B, C, D, E, 4, 4, 16, 256256), qw.QW_ERROR_INVALID_VALUE),     # null qx
    ((A, B, C, D, E, 4, 4, 24, 256256), qw.QW_ERROR_UNSUPPORTED),       # k % 16
    ((A + 8, B, C, D, E, 4, 4, 16, 256256), qw.QW_ERROR_MISALIGNED),    # misaligned qx
])
def test_w8a8_gemm_tile_rejects(args, status):
    assert qw.w8a8_gemm_tile_raw(*args) == status


def test_gemm_tile_empty_is_noop():
    assert qw.w8a16_gemm_tile_raw(0, 0, 0, 0, 0, 0, 0, 0, 0, 4, 16, 256256) == qw.QW_SUCCESS


def test_quantize_empty_is_noop():
    # n == 0: nothing to do, null pointers allowed
    assert qw.quantize_weights_raw(0, 0, 16, 100.0, 0, 0) == qw.QW_SUCCESS


@pytest.mark.parametrize("args,status", [
    ((A, B, C, D, -1, 4, 16), qw.QW_ERROR_INVALID_VALUE),
    ((A, B, C, D, 1, -4, 16), qw.QW_ERROR_INVALID_VALUE),
    ((A, B, C, D, 1, 4, 0), qw.QW_ERROR_INVALID_VALUE),
    ((0, B, C, D, 1, 4, 16), qw.QW_ERROR_INVALID_VALUE),
    ((A, 0, C, D, 1, 4, 16), qw.QW_ERROR_INVALID_VALUE),
    ((A, B, 0, D, 1, 4, 16), qw.QW_ERROR_INVALID_VALUE),
    ((A, B, C, 0, 1, 4, 16), qw.QW_ERROR_INVALID_VALUE),
    ((A, B, C, D, 1, 4, 24), qw.QW_ERROR_UNSUPPORTED),
    ((A, B, C, D, 1 << 31, 4, 16), qw.QW_ERROR_UNSUPPORTED),
    ((A, B, C, D, 1, 1 << 31, 16), qw.QW_ERROR_UNSUPPORTED),
    ((A + 2, B, C, D, 1, 4, 16), qw.QW_ERROR_MISALIGNED),
    ((A, B + 1, C, D, 1, 4, 16), qw.QW_ERROR_MISALIGNED),
    ((A, B, C + 8, D, 1, 4, 16), qw.QW_ERROR_MISALIGNED),
    ((A, B, C, D + 4, 1, 4, 16), qw.QW_ERROR_MISALIGNED),
    ((A, B, C, A + 16, 1, 4, 16), qw.QW_ERROR_INVALID_VALUE),       # y overlaps x
    ((A, B, C, B, 1, 4, 16), qw.QW_ERROR_INVALID_VALUE),            # y overlaps q
    ((A, B, C, C - 16, 2, 8, 16), qw.QW_ERROR_INVALID_VALUE),       # y overlaps scales
])
def test_gemm_rejects(args, status):
    assert qw.w8a16_gemm_raw(*args) == status




@pytest.mark.parametrize("args,status", [
    ((A, B, C, D, E, -1, 4, 16), qw.QW_ERROR_INVALID_VALUE),
    ((A, B, C, D, E, 1, -4, 16), qw.QW_ERROR_INVALID_VALUE),
    ((A, B, C, D, E, 1, 4, 0), qw.QW_ERROR_INVALID_VALUE),
    ((0, B, C, D, E, 1, 4, 16), qw.QW_ERROR_INVALID_VALUE),
    ((A, 0, C, D, E, 1, 4, 16), qw.QW_ERROR_INVALID_VALUE),
    ((A, B, 0, D, E, 1, 4, 16), qw.QW_ERROR_INVALID_VALUE),
    ((A, B, C, 0, E, 1, 4, 16), qw.QW_ERROR_INVALID_VALUE),
    ((A, B, C, D, 0, 1, 4, 16), qw.QW_ERROR_INVALID_VALUE),
    ((A, B, C, D, E, 1, 4, 24), qw.QW_ERROR_UNSUPPORTED),
    ((A, B, C, D, E, 1 << 31, 4, 16), qw.QW_ERROR_UNSUPPORTED),
    ((A, B, C, D, E, 1, 4, 131072 + 16), qw.QW_ERROR_UNSUPPORTED),  # int32 accumulator limit
    ((A + 1, B, C, D, E, 1, 4, 16), qw.QW_ERROR_MISALIGNED),
    ((A, B + 2, C, D, E, 1, 4, 16), qw.QW_ERROR_MISALIGNED),
    ((A, B, C + 8, D, E, 1, 4, 16), qw.QW_ERROR_MISALIGNED),
    ((A, B, C, D + 4, E, 1, 4, 16), qw.QW_ERROR_MISALIGNED),
    ((A, B, C, D, E + 2, 1, 4, 16), qw.QW_ERROR_MISALIGNED),
    ((A, B, C, D, A, 2, 4, 16), qw.QW_ERROR_INVALID_VALUE),         # y overlaps qx
    ((A, B, C, D, B - 16, 2, 8, 16), qw.QW_ERROR_INVALID_VALUE),    # y overlaps sx
    ((A, B, C, D, C + 32, 1, 4, 16), qw.QW_ERROR_INVALID_VALUE),    # y overlaps q
    ((A, B, C, D, D, 1, 4, 16), qw.QW_ERROR_INVALID_VALUE),         # y overlaps scales
])
def test_w8a8_rejects(args, status):
    assert qw.w8a8_gemm_raw(*args) == status


def test_w8a8_auto_path_choice():
    """The int8 kernels share the W8A16 skinny/MFMA crossover (there is no
    W8A8 GEMV)."""
    assert qw.w8a8_auto_path(1, 27392, 4096) == "skinny"
    assert qw.w8a8_auto_path(32, 27392, 4096) == "skinny"
    assert qw.w8a8_auto_path(33, 27392, 4096) == "mfma"
    assert qw.w8a8_auto_path(96, 4608, 4096) == "skinny"
    assert qw.w8a8_auto_path(512, 27392, 4096) == "mfma"
    for m, n, k in ((8, 4608, 4096), (48, 4608, 4096), (200, 4096, 1024), (4096, 4096, 1024)):
        assert qw.w8a8_auto_path(m, n, k) == qw.auto_path(m, n, k)
    assert qw.library().qw_w8a8_gemm_auto_path(8, 64, qw.W8A8_MAX_K + 16) == -1
    with pytest.raises(ValueError):
        qw.w8a8_auto_path(1, 4, 24)


def test_w8a8_empty_is_noop():
    assert qw.w8a8_gemm_raw(0, 0, 0, 0, 0, 0, 4, 16) == qw.QW_SUCCESS
    assert qw.w8a8_gemm_raw(0, 0, 0, 0, 0, 3, 0, 16) == qw.QW_SUCCESS


@pytest.mark.parametrize("args,status", [
    ((A, B, C, D, -1, 4, 16), qw.QW_ERROR_INVALID_VALUE),
    ((0, B, C, D, 1, 4, 16), qw.QW_ERROR_INVALID_VALUE),
    ((A, B, C, D, 1, 4, 24), qw.QW_ERROR_UNSUPPORTED),
    ((A + 2, B, C, D, 1, 4, 16), qw.QW_ERROR_MISALIGNED),
    ((A, B, C, A + 16, 1, 4, 16), qw.QW_ERROR_INVALID_VALUE),       # y overlaps x
])
def test_gemm_tune_rejects(args, status):
    assert qw.w8a16_gemm_tune_raw(*args) == status


def test_tuned_choice_without_records():
    qw.tune_reset()
    assert qw.tuned_choice(8, 4608, 4096) is None
    assert qw.w8a8_tuned_choice(8, 4608, 4096) is None
    assert qw.library().qw_w8a16_gemm_tuned_choice(0, 4, 16) == -1
    assert qw.library().qw_w8a16_gemm_tuned_choice(1, 4, 24) == -1
    assert qw.library().qw_w8a8_gemm_tuned_choice(1, 4, 24) == -1


def test_w8a8_tune_checks_arguments_first():
    # rejected on the host before anything is enqueued; an empty shape is a no-op
    assert qw.w8a8_gemm_tune_raw(A, B, C, D, E, 4, 8, 24) == qw.QW_ERROR_UNSUPPORTED
    assert qw.w8a8_gemm_tune_raw(0, B, C, D, E, 4, 8, 16) == qw.QW_ERROR_INVALID_VALUE
    assert qw.w8a8_gemm_tune_raw(A, B, C, D, E, 4, 8, qw.W8A8_MAX_K + 16) == qw.QW_ERROR_UNSUPPORTED
    assert qw.w8a8_gemm_tune_raw(0, 0, 0, 0, 0, 0, 8, 16) == qw.QW_SUCCESS


def test_gemm_path_checks():
    assert qw.w8a16_gemm_raw(A, B, C, D, 1, 4, 16, 0, 7) == qw.QW_ERROR_INVALID_VALUE
    # the GEMV path refuses shapes beyond its LDS budget: m > 8, or m * ceil(k/1024) > 32
    assert qw.w8a16_gemm_raw(A, B, C, D, 9, 4, 16, 0, 1) == qw.QW_ERROR_UNSUPPORTED
    assert qw.w8a16_gemm_raw(A, B, C, D, 8, 4, 5 * 1024, 0, 1) == qw.QW_ERROR_UNSUPPORTED


def test_auto_path_choice():
    assert qw.auto_path(1, 27392, 4096) == "gemv"
    assert qw.auto_path(8, 4608, 4096) == "skinny"
    assert qw.auto_path(512, 27392, 4096) == "mfma"
    assert qw.auto_path(4096, 4096, 1024) == "mfma"
    # crossover: the skinny kernel while it needs at most 8 passes (16 rows
    # each, 32 for 17..32 rows at k >= 2048) and the passes after the first
    # read at most 128 MiB of weights
    assert qw.auto_path(16, 27392, 4096) == "skinny"
    assert qw.auto_path(24, 27392, 4096) == "skinny"   # one 32-row pass
    assert qw.auto_path(32, 27392, 4096) == "skinny"
    assert qw.auto_path(33, 27392, 4096) == "mfma"     # two more passes over 112 MB
    assert qw.auto_path(24, 27392, 1024) == "skinny"   # 16-row passes at short k: one more over 28 MB
    assert qw.auto_path(128, 4608, 4096) == "skinny"   # seven more passes over 18.9 MB (126 MiB)
    assert qw.auto_path(129, 4608, 4096) == "mfma"     # nine passes
    assert qw.auto_path(128, 4096, 1024) == "skinny"
    assert qw.auto_path(256, 4096, 1024) == "mfma"     # sixteen passes
    # k too long for the GEMV's LDS staging: skinny even at m = 1
    assert qw.auto_path(1, 64, 65536) == "skinny"
    with pytest.raises(ValueError):
        qw.auto_path(1, 4, 24)


def test_mfma_row_length_limit():
    """Rows longer than QW_MFMA_MAX_K: the automatic choice takes the skinny
    kernel, and a forced MFMA path is refused before anything is enqueued."""
    big = qw.MFMA_MAX_K + 16
    assert qw.auto_path(512, 27392, qw.MFMA_MAX_K) == "mfma"
    assert qw.auto_path(512, 27392, big) == "skinny"
    assert qw.library().qw_w8a16_gemm_auto_path(4096, 4096, big) == qw.PATHS["skinny"]
    # fake addresses 1 TiB apart, so that the operands of this size do not overlap
    x, q, s, y = 1 << 40, 2 << 40, 3 << 40, 4 << 40
    assert qw.w8a16_gemm_raw(x, q, s, y, 512, 4, big, 0, qw.PATHS["mfma"]) == qw.QW_ERROR_UNSUPPORTED


def test_header_size_limits_match_the_binding():
    text = open(HEADER).read()
    for name, value in (("QW_QUANTIZE_MAX_K", qw.QUANTIZE_MAX_K), ("QW_MFMA_MAX_K", qw.MFMA_MAX_K),
                        ("QW_W8A8_MAX_K", qw.W8A8_MAX_K)):
        m = re.search(r"#define %s (\d+)" % name, text)
        assert m and int(m.group(1)) == value, name


def test_gemm_empty_is_noop():
    assert qw.w8a16_gemm_raw(0, 0, 0, 0, 0, 4, 16) == qw.QW_SUCCESS
    assert qw.w8a16_gemm_raw(0, 0, 0, 0, 3, 0, 16) == qw.QW_SUCCESS


def test_torch_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        qw.quantize_weights(torch.zeros(4, 16))
    with pytest.raises((TypeError, ValueError)):
        qw.w8a16_gemm(torch.zeros(1, 16), torch.zeros(4, 16, dtype=torch.int8),
                      torch.zeros(4, dtype=torch.float16))


# ---------------------------------------------------------------------------
# Launch failures: a call that passes every host check but cannot be
# enqueued (here: no GPU in the process) reports QW_ERROR_LAUNCH.  The fake
# addresses are never dereferenced because nothing is launched; the test is
# skipped wherever a GPU is visible, where they would reach a kernel.
# ---------------------------------------------------------------------------

def _gpu_visible():
    if os.path.exists("/dev/kfd"):
        return True
    try:
        import torch
        return torch.cuda.device_count() > 0
    except ImportError:
        return False


no_gpu_only = pytest.mark.skipif(_gpu_visible(), reason="valid calls would launch kernels on fake addresses")


@no_gpu_only
def test_valid_calls_without_a_device_report_launch_errors():
    L = qw.QW_ERROR_LAUNCH
    assert qw.quantize_weights_raw(A, 4, 16, 100.0, B, C) == L
    assert qw.quantize_weights_raw(A, 4, 16, 99.0, B, C) == L
    assert qw.quantize_weights_f16_raw(A, 4, 16, 100.0, B, C) == L
    assert qw.quantize_weights_fixed_range_raw(A, 4, 16, D, B, C) == L
    assert qw.quantize_weights_asym_raw(A, 4, 16, B, C, D) == L
    for path in (0, 1, 2, 3):
        assert qw.w8a16_gemm_raw(A, B, C, D, 1, 16, 16, 0, path) == L
        assert qw.w8a16_gemm_asym_raw(A, B, C, E, D, 1, 16, 16, 0, path) == L
    for path in (0, 2, 3):
        assert qw.w8a8_gemm_raw(A, E, B, C, D, 4, 16, 16, 0, path) == L
    assert qw.probe_stream_read_raw(A, 4096, 0, B) == L
    assert qw.probe_shader_clock_raw(A) == L


@pytest.mark.parametrize("args,status", [
    ((A, -1, 0, B), qw.QW_ERROR_INVALID_VALUE),      # negative size
    ((0, 4096, 0, B), qw.QW_ERROR_INVALID_VALUE),    # null buffer
    ((A, 4096, 0, 0), qw.QW_ERROR_INVALID_VALUE),    # null sink
    ((A + 8, 4096, 0, B), qw.QW_ERROR_MISALIGNED),
])
def test_probe_stream_read_rejects(args, status):
    assert qw.probe_stream_read_raw(*args) == status


def test_probe_stream_read_below_one_chunk_is_noop():
    assert qw.probe_stream_read_raw(0, 1023, 0, 0) == qw.QW_SUCCESS


def test_probe_shader_clock_rejects():
    assert qw.probe_shader_clock_raw(0) == qw.QW_ERROR_INVALID_VALUE
    assert qw.probe_shader_clock_raw(A + 4) == qw.QW_ERROR_MISALIGNED

"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them.

Each mutant is a textual edit of ``oracle/qw_oracle.c`` compiled into a
temporary library; the fast pins of ``oracle_pins.py`` then run against it
and at least one must fail.  This is what makes the pins worth trusting: a
pin set that a dropped term, a wrong sign or index, a transposed operand or
a wrong rounding rule would slip through is not a pin set.
"""

import os

import pytest

import oracle
import oracle_pins as P

MUTANTS = {
    # rounding: half away from zero instead of half to even
    "round_half_away": ("float rounded = rintf(ratio);", "float rounded = roundf(ratio);"),
    # reciprocal-multiply instead of true IEEE division
    "reciprocal_multiply": ("float ratio = row[j] / s; ", "float ratio = row[j] * (1.0f / s); "),
    # quantize with the unrounded binary32 scale
    "fp32_scale_for_codes": ("float ratio = row[j] / s; ", "float ratio = row[j] / s32; "),
    # clamp range +-128 on the negative side
    "clamp_minus_128": ("if (rounded < -127.0f)\n            rounded = -127.0f;",
                        "if (rounded < -128.0f)\n            rounded = -128.0f;"),
    # fixed-range clip: bound taken as the row absmax instead of the given one
    "fixed_range_ignores_bound": ("scales[r] = quantize_row_with_bound(w + r * k, k, bounds[r], q + r * k);",
                                  "scales[r] = quantize_row_with_bound(w + r * k, k, (float)oracle_row_percentile(w + r * k, 1, 100.0, (float[1]){0}), q + r * k);"),
    # wrong bound divisor
    "divide_by_128": ("float s32 = t / 127.0f;", "float s32 = t / 128.0f;"),
    # percentile: wrong rank (ceil) and dropped interpolation term
    "percentile_ceil": ("double i_floor = floor(pos);", "double i_floor = ceil(pos);"),
    "percentile_no_interp": ("return lo + step;", "return lo;"),
    "percentile_wrong_neighbour": ("double hi = (double)scratch[i + 1];", "double hi = (double)scratch[k - 1];"),
    # binary16 rounding: ties away, and a wrong subnormal boundary
    "f16_ties_away": ("if (rem > half || (rem == half && (whole & 1)))", "if (rem >= half)"),
    "f16_subnormal_edge": ("int quantum_exp = (lead < -14 ? -14 : lead) - 10;",
                           "int quantum_exp = (lead < -15 ? -15 : lead) - 10;"),
    "f16_decode_bias": ("v = ldexpf((float)(1024 + frac), expfield - 25);",
                        "v = ldexpf((float)(1024 + frac), expfield - 24);"),
    # matmul: dropped scale, wrong sign, transposed/wrong operand index
    "gemm_drops_scale": ("double wdeq = ((double)qrow[j] - z) * s;", "double wdeq = ((double)qrow[j] - z);"),
    "gemm_wrong_sign": ("acc += xv * wdeq;", "acc -= xv * wdeq;"),
    "gemm_reversed_k": ("double xv = (double)oracle_f16_to_f32(xrow[j]);",
                        "double xv = (double)oracle_f16_to_f32(xrow[k - 1 - j]);"),
    "gemm_scale_of_wrong_row": ("ref[i * n + j] = dot_one(x + i * k, q + j * k, 0.0,\n                                     (double)oracle_f16_to_f32(scales[j]), k);",
                                "ref[i * n + j] = dot_one(x + i * k, q + j * k, 0.0,\n                                     (double)oracle_f16_to_f32(scales[i % n]), k);"),
    # outlier-aware quantizer and matmul
    "outliers_at_bound": ("if (fabsf(row[j]) > thresh[r]) {", "if (fabsf(row[j]) >= thresh[r]) {"),
    "outliers_keep_code": ("                q[r * k + j] = 0;\n                ++used;", "                ++used;"),
    "gemm_outliers_dropped": ("acc += xv * (double)val[e];", "acc += 0.0 * xv * (double)val[e];"),
    "gemm_outliers_wrong_column": ("double xv = (double)oracle_f16_to_f32(xrow[idx[e]]);",
                                   "double xv = (double)oracle_f16_to_f32(xrow[e]);"),
    # asymmetric quantizer and matmul
    "asym_divide_by_256": ("float s32 = range / 255.0f;", "float s32 = range / 256.0f;"),
    "asym_range_without_zero": ("float hi = 0.0f, lo = 0.0f;", "float hi = -INFINITY, lo = INFINITY;"),
    "asym_zero_point_unshifted": ("float zf = rintf(-lo / s) - 128.0f;", "float zf = rintf(-lo / s);"),
    "asym_zero_point_sign": ("float c = rintf(row[j] / s) + zf;", "float c = rintf(row[j] / s) - zf;"),
    "asym_round_half_away": ("float c = rintf(row[j] / s) + zf;", "float c = roundf(row[j] / s) + zf;"),
    "asym_clamp_at_127": ("if (c < -128.0f)\n                c = -128.0f;", "if (c < -127.0f)\n                c = -127.0f;"),
    "gemm_asym_zero_point_sign": ("double wdeq = ((double)qrow[j] - z) * s;", "double wdeq = ((double)qrow[j] + z) * s;"),
    "gemm_asym_zero_of_wrong_row": ("const double zj = (double)zeros[j];", "const double zj = (double)zeros[i % n];"),
    # W8A8: dropped activation scale, wrong sign, reversed k, narrow
    # accumulator, activation scale taken from the weight's row index
    "w8a8_drops_x_scale": ("return (double)acc * (sx * sw);", "return (double)acc * sw;"),
    "w8a8_wrong_sign": ("acc += (int64_t)xrow[j] * (int64_t)qrow[j];",
                        "acc -= (int64_t)xrow[j] * (int64_t)qrow[j];"),
    "w8a8_reversed_k": ("acc += (int64_t)xrow[j] * (int64_t)qrow[j];",
                        "acc += (int64_t)xrow[k - 1 - j] * (int64_t)qrow[j];"),
    "w8a8_int16_accumulator": ("    int64_t acc = 0;\n    for (int64_t j = 0; j < k; ++j)\n        acc += (int64_t)xrow[j]",
                               "    int16_t acc = 0;\n    for (int64_t j = 0; j < k; ++j)\n        acc += (int64_t)xrow[j]"),
    "w8a8_x_scale_of_wrong_row": ("w8a8_one(qx + i * k, q + j * k, (double)oracle_f16_to_f32(sx[i]), sw, k);",
                                  "w8a8_one(qx + i * k, q + j * k, (double)oracle_f16_to_f32(sx[j % m]), sw, k);"),
}


@pytest.fixture(scope="module")
def source_text():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, source_text, name):
    old, new = MUTANTS[name]
    assert source_text.count(old) == 1, "mutation site for %s not found exactly once" % name
    src = tmp_path / ("mutant_%s.c" % name)
    src.write_text(source_text.replace(old, new))
    lib_path = str(tmp_path / ("libmutant_%s.so" % name))
    oracle.build(source=str(src), output=lib_path)
    mut = oracle.Oracle(oracle.load_library(lib_path))
    caught = []
    for pin in P.FAST_PINS:
        try:
            pin(mut)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, "mutant %s passed every pin" % name
    os.remove(lib_path)

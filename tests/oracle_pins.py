"""Pins that tie the CPU oracle to something other than itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with what the pages or the mathematics fix:

  * library routines on special cases (torch / numpy binary16 conversion,
    numpy's type-7 percentile on binary64 input, numpy binary64 matmul);
  * brute force with exact rationals (``fractions.Fraction``) on tiny inputs:
    nearest-representable searches for every rounding and Python's
    round-half-to-even on exact quotients;
  * closed forms and invariants (|q| <= 127, the bound element maps to
    +-127, error <= S/2 for unclipped weights, monotonicity, exact scaling);
  * the pages' worked example (bound 0.08 labelled with code 127 on the
    symmetric-quantization slide of the LightSeq deck), stored under
    ``tests/golden/``.

The same functions run against deliberately broken builds of the oracle in
``test_oracle_mutants.py`` to show that each plausible mistake fails at
least one of them.
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------
# exact-rational helpers (independent of the oracle)
# --------------------------------------------------------------------------

def _frac(v) -> Fraction:
    return Fraction(float(v))


def nearest_repr(r: Fraction, dtype):
    """Round the rational r to the nearest value of a numpy float dtype, ties
    to the even significand, by searching the neighbours of a first guess."""
    guess = dtype(float(r))
    if not np.isfinite(guess):
        return guess
    cands = {guess, np.nextafter(guess, dtype(-np.inf)), np.nextafter(guess, dtype(np.inf))}
    best, best_d = None, None
    for c in cands:
        if not np.isfinite(c):
            continue
        d = abs(_frac(c) - r)
        if best is None or d < best_d:
            best, best_d = c, d
        elif d == best_d:
            ib = np.array([best], dtype=dtype).view(np.uint16 if dtype == np.float16 else np.uint32)[0]
            ic = np.array([c], dtype=dtype).view(np.uint16 if dtype == np.float16 else np.uint32)[0]
            if (ic & 1) == 0 and (ib & 1) == 1:
                best = c
    return dtype(best)


def exact_percentile(vals, pct: float) -> Fraction:
    """Type-7 percentile of a list of floats, in exact rationals."""
    a = sorted(_frac(abs(v)) for v in vals)
    k = len(a)
    pos = Fraction(pct) / 100 * (k - 1)
    i = math.floor(pos)
    if i >= k - 1:
        return a[-1]
    f = pos - i
    return a[i] + f * (a[i + 1] - a[i])


def f16_from_bits(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16)


# --------------------------------------------------------------------------
# binary16 conversions
# --------------------------------------------------------------------------

def _torch_f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float16).view(torch.int16).numpy().view(np.uint16)


def check_f32_to_f16_chunk(o, patterns: np.ndarray):
    x = patterns.view(np.float32)
    got = o.f32_to_f16_bits(x)
    want = _torch_f32_to_f16_bits(x)
    nan_in = np.isnan(x)
    fin = ~nan_in
    bad = np.nonzero(got[fin] != want[fin])[0]
    assert bad.size == 0, "fp32->fp16 mismatch at bits %s: got %s want %s" % (
        patterns[fin][bad[:4]], got[fin][bad[:4]], want[fin][bad[:4]])
    # NaN in -> NaN out (payload bits are not part of the contract)
    g = got[nan_in]
    assert np.all(((g & 0x7c00) == 0x7c00) & ((g & 0x3ff) != 0)), "NaN must stay NaN"


def pin_f32_to_f16_sample(o, seed=1):
    """Random bit patterns plus every boundary region of binary16 against
    torch's CPU conversion and numpy's."""
    rng = np.random.default_rng(seed)
    pats = [rng.integers(0, 2**32, size=1 << 18, dtype=np.uint64).astype(np.uint32)]
    # all binary32 values within +-2^12 ulps of every binary16 boundary
    # (each half-ulp point, the subnormal range and overflow)
    h = np.arange(0, 0x7c01, dtype=np.uint16).view(np.float16).astype(np.float32)
    mids = ((h[:-1].astype(np.float64) + h[1:].astype(np.float64)) / 2).astype(np.float32)
    base = np.concatenate([h, mids, np.float32([65504.0, 65520.0, 2.0**-24, 2.0**-25, 2.0**-14])])
    bb = base.view(np.uint32).astype(np.int64)
    offs = np.arange(-3, 4, dtype=np.int64)
    near = (bb[:, None] + offs[None, :]).ravel()
    near = near[(near >= 0) & (near < 0x7f800000)].astype(np.uint32)
    pats.append(near)
    pats.append(near | np.uint32(0x80000000))
    pats = np.concatenate(pats)
    check_f32_to_f16_chunk(o, pats)
    # numpy's own (scalar) conversion on a slice of the same patterns
    x = pats[: 1 << 16].view(np.float32)
    fin = np.isfinite(x)
    assert np.array_equal(o.f32_to_f16_bits(x)[fin], x.astype(np.float16).view(np.uint16)[fin])


def pin_f16_to_f32_exhaustive(o):
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    got = o.f16_bits_to_f32(bits)
    want = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def pin_f64_to_f16(o, seed=2):
    """binary64 -> binary16 directly (no detour through binary32), against
    numpy's direct conversion and against exact nearest search."""
    rng = np.random.default_rng(seed)
    x = np.concatenate([
        rng.standard_normal(1 << 16) * 10.0 ** rng.integers(-9, 6, size=1 << 16),
        # double-rounding traps: just above/below a binary16 half-ulp point by
        # less than a binary32 ulp (a detour through binary32 would round to
        # the tie and then to even)
        (np.arange(1, 2049, dtype=np.float64) + 0.5) * 2.0**-10 * (1 + 2.0**-40),
        (np.arange(1, 2049, dtype=np.float64) + 0.5) * 2.0**-10 * (1 - 2.0**-40),
        np.array([65504.0, 65519.99, 65520.0, 2.0**-24, 2.0**-25, 2.0**-25 * (1 + 2.0**-30), 0.0, -0.0]),
    ])
    got = o.f64_to_f16_bits(x)
    want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want), "fp64->fp16 disagrees with numpy"
    for v in list(x[-8:]) + list(x[:64]):
        r = _frac(v)
        if abs(v) >= 65520.0:
            continue
        assert got[np.nonzero(x == v)[0][0]] == np.array([nearest_repr(r, np.float16)]).view(np.uint16)[0]


# --------------------------------------------------------------------------
# threshold
# --------------------------------------------------------------------------

def pin_percentile_vs_numpy(o, seed=3):
    rng = np.random.default_rng(seed)
    for k in (1, 2, 3, 16, 1024, 4096):
        for pct in (100.0, 99.99, 99.9, 99.0, 90.0, 50.0, 12.5, 0.01):
            row = (rng.standard_normal(k) * 0.02).astype(np.float32)
            got = o.row_percentile(row, pct)
            want = float(np.percentile(np.abs(row).astype(np.float64), pct, method="linear"))
            tol = 4 * np.spacing(np.float64(np.abs(row).max()))
            assert abs(got - want) <= tol, (k, pct, got, want)


def pin_percentile_bruteforce(o, seed=4):
    rng = np.random.default_rng(seed)
    for trial in range(300):
        k = int(rng.integers(1, 12))
        row = (rng.standard_normal(k) * 10.0 ** rng.integers(-3, 2)).astype(np.float32)
        pct = float(rng.choice([100.0, 99.99, 75.0, 50.0, 33.3, 25.0, 1.0, float(rng.uniform(0.001, 100.0))]))
        got = Fraction(o.row_percentile(row, pct))
        want = exact_percentile(row, pct)
        top = _frac(np.abs(row).max())
        assert abs(got - want) <= top * Fraction(1, 2**50), (row, pct, float(got), float(want))
    # exact special cases: median of 5, quartiles, the maximum
    row = np.float32([0.5, -3.0, 2.0, -1.0, 4.0])
    assert o.row_percentile(row, 50.0) == 2.0
    assert o.row_percentile(row, 25.0) == 1.0
    assert o.row_percentile(row, 100.0) == 4.0
    assert abs(o.row_percentile(row, 1e-9) - 0.5) < 1e-9
    assert o.row_percentile(np.float32([1.0, 3.0]), 50.0) == 2.0


# --------------------------------------------------------------------------
# scale and quantizer
# --------------------------------------------------------------------------

def check_scale_rows(t, s_bits, sample=None):
    """s must be the binary16 nearest to the binary32 nearest to t/127."""
    idx = range(len(t)) if sample is None else sample
    for r in idx:
        exact = _frac(t[r]) / 127
        s32 = nearest_repr(exact, np.float32)
        s16 = nearest_repr(_frac(s32), np.float16)
        got = f16_from_bits(s_bits[r:r + 1])[0]
        assert np.array([got]).view(np.uint16)[0] == np.array([s16]).view(np.uint16)[0], (r, t[r], got, s16)


def check_quant_elements(w, q, s_bits, rows=None, cols=None):
    """Brute force per element: q = clamp(round_half_even(fl32(w/S))).
    Returns how many elements the fp32 quotient rounds differently from the
    exact quotient (tie artefacts of the reading; reported, not failed)."""
    artefacts = 0
    s = f16_from_bits(s_bits).astype(np.float32)
    rows = range(w.shape[0]) if rows is None else rows
    for r in rows:
        sr = _frac(s[r])
        cs = range(w.shape[1]) if cols is None else cols
        for c in cs:
            if sr == 0:
                assert q[r, c] == 0
                continue
            exact = _frac(w[r, c]) / sr
            v32 = _frac(nearest_repr(exact, np.float32))
            want = max(-127, min(127, round(v32)))
            want_exact = max(-127, min(127, round(exact)))
            assert int(q[r, c]) == want, (r, c, float(w[r, c]), float(s[r]), int(q[r, c]), want)
            artefacts += int(want != want_exact)
    return artefacts


def pin_scale_and_quantize_bruteforce(o, seed=5):
    rng = np.random.default_rng(seed)
    for trial in range(60):
        n = int(rng.integers(1, 4))
        k = int(rng.integers(1, 24))
        w = (rng.standard_normal((n, k)) * 10.0 ** rng.integers(-4, 2)).astype(np.float32)
        if trial % 5 == 0:
            # exact ties: values that are (j + 1/2) * S for a power-of-two S
            w[:, : min(k, 4)] = np.float32([0.5, 1.5, 2.5, -2.5][: min(k, 4)]) * np.float32(2.0**-8)
            w[:, -1] = np.float32(127 * 2.0**-8)
        pct = float(rng.choice([100.0, 99.0, 90.0, 50.0]))
        q, s, t = o.quantize(w, pct)
        for r in range(n):
            want_t = np.float32(float(exact_percentile(w[r], pct)))
            # the bound is the binary32 rounding of the binary64 interpolation
            assert abs(_frac(t[r]) - exact_percentile(w[r], pct)) <= _frac(np.spacing(want_t)), (w[r], pct, t[r])
        check_scale_rows(t, s)
        check_quant_elements(w, q, s)


def pin_quantize_exact_ties(o, seed=11):
    """Rows whose scale is a chosen binary16 value S (the row bound is 127*S,
    exact) and whose other weights sit exactly on (j + 1/2) * S: the exact
    quotient is a tie, which must go to the even code.  Non-power-of-two S
    make 1/S inexact, so a reciprocal-multiply quotient lands beside the tie."""
    rng = np.random.default_rng(seed)
    js = np.arange(-127, 127, dtype=np.float64)
    for trial in range(8):
        s_target = np.float16(rng.uniform(3e-4, 1e-3))
        sv = float(s_target)
        row = np.concatenate([(js + 0.5) * sv, [127.0 * sv]]).astype(np.float32)
        assert np.all(row.astype(np.float64) == np.concatenate([(js + 0.5) * sv, [127.0 * sv]]))
        q, s, t = o.quantize(row[None, :], 100.0)
        assert s[0] == np.array([s_target]).view(np.uint16)[0]
        want = np.array([max(-127, min(127, round(Fraction(2 * int(j) + 1, 2)))) for j in js] + [127])
        assert np.array_equal(q[0].astype(np.int64), want), np.nonzero(q[0] != want)


def pin_page_example(o):
    """The symmetric-quantization slide labels the bound 0.08 with code 127."""
    with open(os.path.join(GOLDEN, "symmetric_bound_example.json")) as f:
        ex = json.load(f)
    bound, code = np.float32(ex["bound"]), int(ex["max_code"])
    row = np.float32([[bound, -bound / 2, bound / 4, 0.0, -bound]])
    q, s, t = o.quantize(row, 100.0)
    assert t[0] == bound
    assert int(q[0, 0]) == code and int(q[0, 4]) == -code
    sv = float(f16_from_bits(s)[0])
    assert abs(float(bound) - code * sv) <= sv / 2
    check_scale_rows(t, s)
    check_quant_elements(row, q, s)


def check_invariants(w, q, s_bits, t, pct):
    """Invariants that hold on any input for the reading taken."""
    s = f16_from_bits(s_bits).astype(np.float32)
    assert q.dtype == np.int8
    assert int(q.min()) >= -127 and int(q.max()) <= 127, "codes outside +-127"
    absw = np.abs(w)
    # sign preserved (or zero)
    assert not np.any((np.sign(q) * np.sign(w)) < 0), "sign flipped"
    # monotone in w within every row
    order = np.argsort(w, axis=1, kind="stable")
    qs = np.take_along_axis(q, order, axis=1).astype(np.int32)
    assert np.all(np.diff(qs, axis=1) >= 0), "not monotone"
    normal = s >= np.float32(2.0**-14)
    # error <= S/2 (plus the binary32 quotient rounding) for unclipped weights
    unclipped = absw <= t[:, None]
    err = np.abs(w.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    bound = s[:, None].astype(np.float64) * (0.5 + 2.0**-17)
    viol = unclipped & (err > bound) & normal[:, None]
    assert not viol.any(), "dequant error above S/2 at %s" % (np.argwhere(viol)[:4],)
    # every weight at or beyond the bound saturates
    big = (absw >= t[:, None]) & (t[:, None] > 0) & normal[:, None]
    assert np.all(np.abs(q[big].astype(np.int32)) == 127), "bound element not +-127"
    if pct == 100.0:
        # the absmax element maps to +-127 with its own sign
        am = np.argmax(absw, axis=1)
        rows = np.nonzero(normal)[0]
        qa = q[rows, am[rows]].astype(np.int32)
        wa = w[rows, am[rows]]
        assert np.all(qa == np.where(wa > 0, 127, -127))
        assert np.array_equal(t, absw.max(axis=1)), "pct=100 must be the absmax"


def pin_quantize_invariants(o, seed=6):
    import synthetic
    for name, pct in (("tiny_m1_k256_n512", 100.0),
                      ("transformer_big_ffn_outliers_m4096_k1024_n4096", 99.99)):
        wl = synthetic.BY_NAME[name]
        _, w = synthetic.make_inputs(wl)
        w = w[:512]
        q, s, t = o.quantize(w, pct)
        check_invariants(w, q, s, t, pct)
        check_scale_rows(t, s, sample=range(0, w.shape[0], 37))
        check_quant_elements(w, q, s, rows=range(0, w.shape[0], 97), cols=range(0, w.shape[1], 13))


def pin_degenerate_rows(o):
    k = 32
    w = np.zeros((6, k), dtype=np.float32)
    w[1, 5] = -3.0e-3                      # a single non-zero
    w[2, :] = 7.0e-2                       # all equal
    w[3, :4] = np.float32(1e-9)            # scale underflows binary16 -> S = 0
    w[4, :] = np.float32(2.0**-10)         # subnormal binary16 scale
    w[4, ::3] = -np.float32(3 * 2.0**-12)
    w[5, 0] = np.float32(1.0e7)            # scale overflows binary16 -> S = inf, q = 0
    w[5, 1] = np.float32(1.0)
    q, s, t = o.quantize(w, 100.0)
    assert np.all(q[0] == 0) and s[0] == 0
    assert q[1, 5] == -127 and np.count_nonzero(q[1]) == 1
    assert np.all(q[2] == 127)
    assert s[3] == 0 and np.all(q[3] == 0)
    assert 0 < s[4] < 0x0400  # subnormal binary16 scale
    check_scale_rows(t, s)
    check_quant_elements(w[:5], q[:5], s[:5])
    assert s[5] == 0x7c00 and np.all(q[5] == 0)


# --------------------------------------------------------------------------
# matmul reference
# --------------------------------------------------------------------------

def pin_gemm_vs_numpy(o, seed=7):
    rng = np.random.default_rng(seed)
    for (m, n, k) in ((1, 5, 16), (3, 17, 48), (9, 33, 80), (16, 64, 256)):
        x = rng.standard_normal((m, k)).astype(np.float16)
        q = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
        s = (rng.uniform(1e-4, 1e-3, size=n)).astype(np.float16).view(np.uint16)
        ref = o.gemm(x, q, s)
        wd = q.astype(np.float64) * f16_from_bits(s).astype(np.float64)[:, None]
        want = x.astype(np.float64) @ wd.T
        tol = 1e-12 * max(1.0, np.abs(want).max())
        assert np.abs(ref - want).max() <= tol
        mi = rng.integers(0, m, size=11)
        ni = rng.integers(0, n, size=11)
        assert np.array_equal(o.gemm_sampled(x, q, s, mi, ni), ref[mi, ni])


def pin_gemm_exact(o, seed=8):
    """X in {-1,0,1}, power-of-two scales: every product and partial sum is
    exact, so the reference equals the integer sum times the scale."""
    rng = np.random.default_rng(seed)
    m, n, k = 5, 40, 512
    x = rng.integers(-1, 2, size=(m, k)).astype(np.float16)
    q = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    e = rng.integers(0, 11, size=n)
    s = (2.0 ** (-e)).astype(np.float16).view(np.uint16)
    ref = o.gemm(x, q, s)
    isum = x.astype(np.int64) @ q.astype(np.int64).T
    want = np.ldexp(isum.astype(np.float64), -e[None, :])
    assert np.array_equal(ref, want)


def pin_gemm_bruteforce(o, seed=9):
    rng = np.random.default_rng(seed)
    for trial in range(20):
        m, n, k = (int(v) for v in rng.integers(1, 5, size=3))
        x = rng.standard_normal((m, k)).astype(np.float16)
        q = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
        s = rng.uniform(1e-4, 1e-2, size=n).astype(np.float16).view(np.uint16)
        ref = o.gemm(x, q, s)
        sv = f16_from_bits(s)
        for i in range(m):
            for j in range(n):
                exact = sum(_frac(x[i, c]) * int(q[j, c]) * _frac(sv[j]) for c in range(k))
                assert abs(_frac(ref[i, j]) - exact) <= Fraction(k) * abs(exact) * Fraction(1, 2**52) + Fraction(1, 2**80)


def pin_gemm_zero_and_scaling(o, seed=10):
    rng = np.random.default_rng(seed)
    m, n, k = 4, 24, 64
    x = rng.standard_normal((m, k)).astype(np.float16)
    q = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    s = rng.uniform(1e-4, 1e-3, size=n).astype(np.float16)
    ref = o.gemm(x, q, s.view(np.uint16))
    zero = o.gemm(np.zeros_like(x), q, s.view(np.uint16))
    assert np.all(zero == 0.0) and not np.any(np.signbit(zero))
    s2 = (s.astype(np.float32) * 2).astype(np.float16)
    ref2 = o.gemm(x, q, s2.view(np.uint16))
    assert np.array_equal(ref2, 2.0 * ref)
    # a column is linear in its own scale only
    assert np.array_equal(o.gemm(x, q[:1], s[:1].view(np.uint16))[:, 0], ref[:, 0])


def _cosine_vs_unquantized(o, name, rows=None):
    import synthetic
    wl = synthetic.BY_NAME[name]
    x, w = synthetic.make_inputs(wl)
    if rows is not None:
        x = x[:rows]
    q, s, _ = o.quantize(w, wl.clip_percentile)
    ref = o.gemm(x, q, s).ravel()
    full = (x.astype(np.float64) @ w.astype(np.float64).T).ravel()
    return float(ref @ full / (np.linalg.norm(ref) * np.linalg.norm(full)))


def pin_cosine_vs_unquantized(o):
    """The W8A16 output stays above 0.99 cosine similarity to the
    unquantized product (ChatGLM2/BM1684X page, section 2), on the tiny,
    the small-batch and the FFN workload (the FFN with its 99.99th
    percentile clip, on its first 256 activation rows).  A dropped scale,
    a wrong row's scale or a transposed operand falls far below."""
    for name, rows in (("tiny_m1_k256_n512", None), ("small_batch_m8_k4096_n4608", None),
                       ("transformer_big_ffn_outliers_m4096_k1024_n4096", 256)):
        cos = _cosine_vs_unquantized(o, name, rows)
        assert cos > 0.99, (name, cos)


def pin_page_matmul_sizes(o):
    """ChatGLM2/BM1684X page, section 3 (TPU-MLIR实现): the right operand of
    one ChatGLM2 MatMul, 4096 x 27392, is 214 MB in F16 and 107 MB after
    int8 quantization (MB read as MiB, truncated; fixture
    tests/golden/chatglm2_matmul_sizes.json).  The oracle's codes for a
    weight of that shape take exactly N * K bytes, one per weight, and its
    scales one binary16 per output row."""
    import json
    import os
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                           "chatglm2_matmul_sizes.json"), encoding="utf-8") as f:
        g = json.load(f)
    n, k = g["n"], g["k"]
    w = np.zeros((n, k), dtype=np.float32)
    w[:, 0] = 0.02  # every row gets a nonzero scale
    q, s, _ = o.quantize(w, 100.0)
    assert q.dtype == np.int8 and q.shape == (n, k)
    assert (q.nbytes >> 20) == g["int8_mb"]
    assert ((2 * n * k) >> 20) == g["f16_mb"]
    assert s.dtype == np.uint16 and s.shape == (n,)
    # the page's 4096-entry scale (0.008 MB) is one per K column, the
    # recorded conflict: one per output row is N entries
    assert abs(g["page_scale_count"] * 2 / 1e6 - g["page_scale_mb"]) < 5e-4
    assert s.nbytes == 2 * n
    assert np.all(q[:, 0] == 127) and np.all(q[:, 1:] == 0)



# --------------------------------------------------------------------------
# fixed-range clip
# --------------------------------------------------------------------------

def pin_fixed_range_bruteforce(o, seed=15):
    """Given bounds (below, at and above the row's absmax, and zero): the
    scale is the binary16 nearest to the binary32 nearest to t/127 and every
    code is the clamped round-half-even of the binary32 quotient, checked
    with exact rationals; elements beyond the bound saturate with their
    sign."""
    rng = np.random.default_rng(seed)
    for trial in range(40):
        n = int(rng.integers(1, 5))
        k = int(rng.integers(1, 20))
        w = (rng.standard_normal((n, k)) * 10.0 ** rng.integers(-3, 2)).astype(np.float32)
        amax = np.abs(w).max(axis=1)
        factor = rng.choice([0.0, 0.3, 0.8, 1.0, 1.7], size=n)
        bounds = (amax * factor).astype(np.float32)
        q, sb = o.quantize_fixed(w, bounds)
        check_scale_rows(bounds, sb)
        check_quant_elements(w, q, sb)
        s = f16_from_bits(sb).astype(np.float64)
        for r in range(n):
            if s[r] == 0:
                assert np.all(q[r] == 0)
                continue
            big = np.abs(w[r].astype(np.float64)) >= 127.5 * s[r]
            assert np.all(np.abs(q[r][big]) == 127)
            assert np.all(np.sign(q[r][big]) == np.sign(w[r][big]))


def pin_fixed_range_of_measured_bound(o, seed=16):
    """With each row's own measured bound (absmax or percentile) passed as
    the fixed range, the result equals the data-driven quantizer's."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((9, 300)) * 0.02).astype(np.float32)
    for pct in (100.0, 99.0, 75.0):
        q, s, t = o.quantize(w, pct)
        qf, sf = o.quantize_fixed(w, t)
        assert np.array_equal(q, qf) and np.array_equal(s, sf)


# --------------------------------------------------------------------------
# outlier-aware quantizer and matmul
# --------------------------------------------------------------------------

def _capacity(k, pct):
    if pct == 100.0:
        return 0
    i = math.floor((pct / 100.0) * (k - 1))
    return 0 if i >= k - 1 else k - 1 - i


def pin_outliers_split(o, seed=20):
    """The side list holds exactly the elements above the (pinned) clip
    bound, in ascending column order with their exact values; their codes are
    0 and every other code is the clipped quantizer's; the slot count never
    exceeds k - 1 - floor(pos)."""
    rng = np.random.default_rng(seed)
    for (n, k, pct) in ((6, 1024, 99.99), (5, 4096, 99.9), (7, 48, 90.0), (4, 64, 100.0), (3, 33, 50.0)):
        w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
        hit = rng.choice(n * k, size=max(1, n * k // 1000), replace=False)
        w.flat[hit] = (rng.standard_normal(hit.size) * 0.2).astype(np.float32)
        w[0, : min(k, 8)] = w[0, 0]  # ties at the top of a row
        cap = _capacity(k, pct)
        assert o.outlier_capacity(k, pct) == cap
        q, sb, idx, val = o.quantize_outliers(w, pct)
        q0, s0, t = o.quantize(w, pct)
        assert np.array_equal(sb, s0)
        for r in range(n):
            if f16_from_bits(sb[r:r + 1])[0] == 0:
                assert np.all(idx[r] == -1)
                continue
            cols = np.nonzero(np.abs(w[r]) > t[r])[0]
            assert len(cols) <= cap
            used = idx[r][idx[r] >= 0]
            assert np.array_equal(used, cols), (r, used, cols)
            assert np.all(idx[r][len(cols):] == -1) and np.all(val[r][len(cols):] == 0.0)
            assert np.array_equal(val[r][: len(cols)], w[r][cols])
            assert np.all(q[r][cols] == 0)
            keep = np.ones(k, bool)
            keep[cols] = False
            assert np.array_equal(q[r][keep], q0[r][keep])
    if _capacity(64, 90.0) > 0:
        w = np.linspace(-1, 1, 4 * 64, dtype=np.float32).reshape(4, 64)
        try:
            o.quantize_outliers(w, 90.0, cap=_capacity(64, 90.0) - 1)
        except ValueError:
            pass
        else:
            raise AssertionError("too few slots must be rejected")


def pin_gemm_outliers(o, seed=21):
    """The reference is the (pinned) dense W8A16 reference plus the side
    list's products (numpy binary64), and exact on exact inputs."""
    rng = np.random.default_rng(seed)
    m, n, k, cap = 5, 24, 256, 3
    x = rng.standard_normal((m, k)).astype(np.float16)
    q = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    s = rng.uniform(1e-4, 1e-2, size=n).astype(np.float16).view(np.uint16)
    idx = np.full((n, cap), -1, dtype=np.int32)
    val = np.zeros((n, cap), dtype=np.float32)
    for r in range(n):
        c = int(rng.integers(0, cap + 1))
        idx[r, :c] = np.sort(rng.choice(k, size=c, replace=False))
        val[r, :c] = rng.standard_normal(c) * 0.5
    ref = o.gemm_outliers(x, q, s, idx, val)
    side = np.zeros((m, n))
    xd = x.astype(np.float64)
    for r in range(n):
        for e in range(cap):
            if idx[r, e] >= 0:
                side[:, r] += xd[:, idx[r, e]] * float(val[r, e])
    want = o.gemm(x, q, s) + side
    assert np.abs(ref - want).max() <= 1e-12 * max(1.0, np.abs(want).max())
    mi = rng.integers(0, m, size=19)
    ni = rng.integers(0, n, size=19)
    assert np.array_equal(o.gemm_outliers_sampled(x, q, s, idx, val, mi, ni), ref[mi, ni])
    xi = rng.integers(-1, 2, size=(m, k)).astype(np.float16)
    e = rng.integers(0, 11, size=n)
    sp = (2.0 ** (-e)).astype(np.float16).view(np.uint16)
    vd = (rng.integers(-512, 512, size=(n, cap)) / 64.0).astype(np.float32)
    vd[idx < 0] = 0.0
    ref2 = o.gemm_outliers(xi, q, sp, idx, vd)
    dense = np.ldexp((xi.astype(np.int64) @ q.astype(np.int64).T).astype(np.float64), -e[None, :])
    side2 = np.zeros((m, n))
    for r in range(n):
        for c in range(cap):
            if idx[r, c] >= 0:
                side2[:, r] += xi[:, idx[r, c]].astype(np.float64) * float(vd[r, c])
    assert np.array_equal(ref2, dense + side2)


# --------------------------------------------------------------------------
# asymmetric (zero-point) quantizer and matmul
# --------------------------------------------------------------------------

def _asym_rows(rng, n, k):
    w = (rng.standard_normal((n, k)) * 10.0 ** rng.integers(-3, 2)).astype(np.float32)
    kind = rng.integers(0, 4)
    if kind == 1:
        w = np.abs(w)                       # all >= 0: lo = 0, z = -128
    elif kind == 2:
        w = -np.abs(w)                      # all <= 0: hi = 0
    elif kind == 3:
        w = (w + np.float32(3.0) * np.abs(w).max()).astype(np.float32)  # offset range
    return w


def pin_asym_quantize_bruteforce(o, seed=17):
    """Exact rationals: the range [min(0, min w), max(0, max w)] in binary32,
    S the binary16 nearest to the binary32 nearest to range/255, z the
    half-even rounding of the binary32 quotient -lo/S shifted by -128, each
    code the half-even rounding of the binary32 quotient w/S plus z, all
    clamped to int8."""
    rng = np.random.default_rng(seed)
    for trial in range(50):
        n = int(rng.integers(1, 4))
        k = int(rng.integers(1, 20))
        w = _asym_rows(rng, n, k)
        if trial % 7 == 0:
            w[0] = 0.0
        if trial % 5 == 1:
            # range 255/256 gives S = 2^-8 exactly; the other weights sit on
            # exact ties (j + 1/2) * S of the quotient
            ties = np.float32([0.5, -0.49609375, 2.5 / 256, -3.5 / 256, 4.5 / 256, 0.5 / 256, -0.5 / 256,
                               6.5 / 256])
            w = np.tile(ties, (n, 1))
            k = w.shape[1]
        q, sb, z = o.quantize_asym(w)
        for r in range(n):
            hi = max(Fraction(0), max(_frac(v) for v in w[r]))
            lo = min(Fraction(0), min(_frac(v) for v in w[r]))
            rng32 = nearest_repr(hi - lo, np.float32)
            s32 = nearest_repr(_frac(rng32) / 255, np.float32)
            s16 = nearest_repr(_frac(s32), np.float16)
            assert sb[r] == np.array([s16]).view(np.uint16)[0], (r, w[r], sb[r], s16)
            S = _frac(s16)
            if S == 0:
                assert z[r] == 0 and np.all(q[r] == 0)
                continue
            zq = round(_frac(nearest_repr(-lo / S, np.float32)))
            zz = max(-128, min(127, zq - 128))
            assert int(z[r]) == zz, (r, int(z[r]), zz)
            for c in range(k):
                v = _frac(nearest_repr(_frac(w[r, c]) / S, np.float32))
                want = max(-128, min(127, round(v) + zz))
                assert int(q[r, c]) == want, (r, c, float(w[r, c]), int(q[r, c]), want)


def pin_asym_quantize_invariants(o, seed=18):
    """Zero maps to the zero point; the row minimum (when negative) maps to
    -128; codes are monotone in w; every weight below the top code is
    recovered to within S/2 (plus the binary32 quotient's rounding)."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((16, 333)) * 0.02).astype(np.float32)
    w[3] = np.abs(w[3]) + np.float32(0.01)
    w[5] = -np.abs(w[5])
    w[:, 7] = 0.0
    q, sb, z = o.quantize_asym(w)
    s = f16_from_bits(sb).astype(np.float64)
    for r in range(w.shape[0]):
        assert q[r, 7] == z[r]
        if w[r].min() < 0 and -128 < z[r] < 127:
            assert q[r, np.argmin(w[r])] == -128
        order = np.argsort(w[r], kind="stable")
        assert np.all(np.diff(q[r][order].astype(np.int32)) >= 0)
        inner = q[r] < 127
        err = np.abs(w[r].astype(np.float64) - s[r] * (q[r].astype(np.float64) - z[r]))[inner]
        assert np.all(err <= s[r] * (0.5 + 2.0 ** -15)), (r, err.max() / s[r])


def pin_gemm_asym(o, seed=19):
    """With zero points 0 the asymmetric reference is the (pinned) symmetric
    one; with X in {-1,0,1} and power-of-two scales every term is exact and it
    equals numpy's int64 product of X and (q - z), scaled."""
    rng = np.random.default_rng(seed)
    m, n, k = 4, 30, 200
    x = rng.standard_normal((m, k)).astype(np.float16)
    q = rng.integers(-128, 128, size=(n, k)).astype(np.int8)
    s = rng.uniform(1e-4, 1e-2, size=n).astype(np.float16).view(np.uint16)
    assert np.array_equal(o.gemm_asym(x, q, s, np.zeros(n, np.int8)), o.gemm(x, q, s))
    xi = rng.integers(-1, 2, size=(m, k)).astype(np.float16)
    z = rng.integers(-128, 128, size=n).astype(np.int8)
    e = rng.integers(0, 11, size=n)
    sp = (2.0 ** (-e)).astype(np.float16).view(np.uint16)
    ref = o.gemm_asym(xi, q, sp, z)
    want = xi.astype(np.int64) @ (q.astype(np.int64) - z.astype(np.int64)[:, None]).T
    assert np.array_equal(ref, np.ldexp(want.astype(np.float64), -e[None, :]))
    mi = rng.integers(0, m, size=17)
    ni = rng.integers(0, n, size=17)
    assert np.array_equal(o.gemm_asym_sampled(xi, q, sp, z, mi, ni), ref[mi, ni])


# --------------------------------------------------------------------------
# W8A8 matmul reference
# --------------------------------------------------------------------------

def pin_w8a8_unit_scales_is_integer_matmul(o, seed=12):
    """With every scale 1.0 the W8A8 reference is the integer matrix product,
    which numpy computes exactly in int64."""
    rng = np.random.default_rng(seed)
    one = np.float16(1.0).view(np.uint16)
    for (m, n, k) in ((1, 3, 16), (5, 7, 33), (4, 9, 1040)):
        qx = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
        q = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
        ref = o.w8a8_gemm(qx, np.full(m, one, np.uint16), q, np.full(n, one, np.uint16))
        want = qx.astype(np.int64) @ q.astype(np.int64).T
        assert np.array_equal(ref, want.astype(np.float64))


def pin_w8a8_equals_w8a16_on_exact_activations(o, seed=13):
    """Power-of-two activation scales make x = qx * Sx exact in binary16, and
    then every term and partial sum of both references is exact, so the W8A8
    reference must equal the (separately pinned) W8A16 reference of the
    dequantized activations exactly, element by element."""
    rng = np.random.default_rng(seed)
    for (m, n, k) in ((3, 5, 48), (6, 11, 256)):
        qx = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
        ex = rng.integers(0, 11, size=m)
        sx = (2.0 ** (-ex)).astype(np.float16)
        x = (qx.astype(np.float64) * sx.astype(np.float64)[:, None]).astype(np.float16)
        assert np.array_equal(x.astype(np.float64), qx.astype(np.float64) * sx.astype(np.float64)[:, None])
        q = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
        s = rng.uniform(1e-4, 1e-2, size=n).astype(np.float16).view(np.uint16)
        ref = o.w8a8_gemm(qx, sx.view(np.uint16), q, s)
        assert np.array_equal(ref, o.gemm(x, q, s))
        mi = rng.integers(0, m, size=13)
        ni = rng.integers(0, n, size=13)
        assert np.array_equal(o.w8a8_gemm_sampled(qx, sx.view(np.uint16), q, s, mi, ni), ref[mi, ni])


def pin_w8a8_scaling_and_symmetry(o, seed=14):
    """Row m scales with Sx[m] alone, column n with S[n] alone, and swapping
    the operands transposes the result."""
    rng = np.random.default_rng(seed)
    m, n, k = 4, 6, 80
    qx = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
    q = rng.integers(-127, 128, size=(n, k)).astype(np.int8)
    sx = rng.uniform(1e-3, 1e-1, size=m).astype(np.float16)
    s = rng.uniform(1e-4, 1e-2, size=n).astype(np.float16)
    ref = o.w8a8_gemm(qx, sx.view(np.uint16), q, s.view(np.uint16))
    sx2 = sx.copy()
    sx2[1] = sx[1] * np.float16(2)
    ref2 = o.w8a8_gemm(qx, sx2.view(np.uint16), q, s.view(np.uint16))
    assert np.array_equal(ref2[1], 2.0 * ref[1])
    assert np.array_equal(np.delete(ref2, 1, 0), np.delete(ref, 1, 0))
    s2 = s.copy()
    s2[4] = s[4] * np.float16(4)
    ref3 = o.w8a8_gemm(qx, sx.view(np.uint16), q, s2.view(np.uint16))
    assert np.array_equal(ref3[:, 4], 4.0 * ref[:, 4])
    assert np.array_equal(np.delete(ref3, 4, 1), np.delete(ref, 4, 1))
    assert np.array_equal(o.w8a8_gemm(q, s.view(np.uint16), qx, sx.view(np.uint16)), ref.T)
    zero = o.w8a8_gemm(np.zeros_like(qx), sx.view(np.uint16), q, s.view(np.uint16))
    assert np.all(zero == 0.0) and not np.any(np.signbit(zero))


FAST_PINS = (
    pin_f32_to_f16_sample,
    pin_f16_to_f32_exhaustive,
    pin_f64_to_f16,
    pin_percentile_vs_numpy,
    pin_percentile_bruteforce,
    pin_scale_and_quantize_bruteforce,
    pin_quantize_exact_ties,
    pin_page_example,
    pin_quantize_invariants,
    pin_degenerate_rows,
    pin_gemm_vs_numpy,
    pin_gemm_exact,
    pin_gemm_bruteforce,
    pin_gemm_zero_and_scaling,
    pin_cosine_vs_unquantized,
    pin_page_matmul_sizes,
    pin_fixed_range_bruteforce,
    pin_fixed_range_of_measured_bound,
    pin_outliers_split,
    pin_gemm_outliers,
    pin_asym_quantize_bruteforce,
    pin_asym_quantize_invariants,
    pin_gemm_asym,
    pin_w8a8_unit_scales_is_integer_matmul,
    pin_w8a8_equals_w8a16_on_exact_activations,
    pin_w8a8_scaling_and_symmetry,
)

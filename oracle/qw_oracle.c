/*
 * qw_oracle.c -- plain, slow CPU oracle for int8 weight-only (W8A16)
 * quantization of Linear weights and the W8A16 matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links
 * or includes this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load it (through oracle/__init__.py).  It
 * shares no code, header, table or constant with the HIP path.
 *
 * What it computes (the method, restated):
 *   - Symmetric linear quantization to n = 8 bits: a per-row bound is mapped
 *     onto the largest code 2^(n-1)-1 = 127, q = round(w / S), and a product
 *     of two such values carries no zero-point cross terms.  Source: LightSeq
 *     slide deck "LightSeq：高性能NLP序列推理实践", slide "量化：裁剪+对称"
 *     (symmetric quantization formula).
 *   - The bound is the row's largest |w|, or a clipped bound (a percentage
 *     clip) when a percentile below 100 is requested.  Source: same deck,
 *     slide "量化流程" (fixed range clip vs percentage clip).
 *   - Weight-only W8A16: Linear weights are stored int8 with one scale per
 *     output channel and dequantized back to F16 for the matmul.  Source:
 *     "探索ChatGLM2在算能BM1684X上INT8量化部署" (elecfans), section 2
 *     (量化方案) and section 3 (TPU-MLIR实现: weight is the right operand,
 *     F16 scale).
 *   - The matmul: load, cast int8 -> F16, multiply by the scale
 *     (dequantize), multiply with the activation, store.  Source: same page,
 *     section 4 (后端性能提升原理), its five-step list.
 *   - Simulation style: low-precision values are carried in a wider float
 *     type and every quantization step is applied explicitly after a
 *     high-precision operation.  Source: QPyTorch review (nubint.ai),
 *     section 提出的方法.
 *
 * Readings taken where the pages leave a step open (each also listed in
 * the design notes):
 *   R1 one scale per output row n of W[N,K] (the weight's output channel);
 *   R2 the clip bound is the linear-interpolated (Hyndman-Fan type 7)
 *      percentile of |w| over the row, interpolated in binary64;
 *   R3 scale S = fp16_RNE( fp32( t / 127 ) ), and quantization divides by
 *      the *stored* fp16 scale;
 *   R4 q = clamp( round_half_even( fp32( w / S ) ), -127, 127 ), true IEEE
 *      binary32 division; S == 0 gives q = 0;
 *   R5 the matmul reference is exact-as-possible binary64:
 *      ref[m][n] = sum_k x[m][k] * (q[n][k] * S[n]);
 *   R6 W8A8 quantizes each activation row with the same quantizer (its
 *      absmax bound) and scales the exact integer product by Sx[m] * S[n].
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -shared
 * -fPIC.  No FMA contraction anywhere; every operation is one IEEE op.
 */
#include <math.h>
#include <stdint.h>
#if defined(_OPENMP)
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

#if defined(__FAST_MATH__)
#error "the oracle must not be built with fast-math"
#endif

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 conversions, written from the format definition:       */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; subnormals have */
/* quantum 2^-24; the largest finite value is 65504; rounding is to nearest */
/* with ties to even.                                                       */
/* ------------------------------------------------------------------------ */

/* Round the non-negative finite value  sig * 2^e  (sig > 0 an integer of at
 * most 63 bits) to binary16 and return the magnitude bits. */
static uint16_t half_from_scaled(uint64_t sig, int e)
{
    /* exponent of the leading bit: |v| in [2^lead, 2^(lead+1)) */
    int nbits = 64 - __builtin_clzll(sig);
    int lead = nbits - 1 + e;
    /* the binary16 quantum (unit in the last place) at this magnitude */
    int quantum_exp = (lead < -14 ? -14 : lead) - 10;
    int shift = quantum_exp - e; /* v / quantum = sig * 2^(-shift) */
    uint64_t n;
    if (shift <= 0) {
        n = sig << (-shift); /* exact; only when v is a small multiple of the quantum */
    } else if (shift > 63) {
        n = 0; /* v < quantum / 2 for sure */
    } else {
        uint64_t whole = sig >> shift;
        uint64_t rem = sig & ((((uint64_t)1) << shift) - 1);
        uint64_t half = ((uint64_t)1) << (shift - 1);
        if (rem > half || (rem == half && (whole & 1)))
            whole += 1;
        n = whole;
    }
    if (lead < -14) {
        /* subnormal range: the bits are the quantum count; a count of 1024
         * is exactly the smallest normal number 0x0400 */
        return (uint16_t)n;
    }
    /* normal range: n in [1024, 2048] */
    int biased = lead + 15;
    if (n == 2048) {
        n = 1024;
        biased += 1;
    }
    if (biased >= 31)
        return 0x7c00; /* overflow to infinity */
    return (uint16_t)((biased << 10) | (int)(n - 1024));
}

uint16_t oracle_f32_to_f16(float x)
{
    uint32_t b;
    memcpy(&b, &x, sizeof b);
    uint16_t sign = (uint16_t)((b >> 16) & 0x8000u);
    uint32_t mag = b & 0x7fffffffu;
    if (mag >= 0x7f800000u) /* inf or nan */
        return (uint16_t)(sign | (mag == 0x7f800000u ? 0x7c00u : 0x7e00u));
    if (mag == 0)
        return sign;
    uint32_t expfield = mag >> 23;
    uint64_t sig = mag & 0x7fffffu;
    int e;
    if (expfield == 0) {
        e = -149; /* binary32 subnormal: sig * 2^-149 */
    } else {
        sig |= 0x800000u;
        e = (int)expfield - 150;
    }
    return (uint16_t)(sign | half_from_scaled(sig, e));
}

uint16_t oracle_f64_to_f16(double x)
{
    uint64_t b;
    memcpy(&b, &x, sizeof b);
    uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
    uint64_t mag = b & 0x7fffffffffffffffull;
    if (mag >= 0x7ff0000000000000ull)
        return (uint16_t)(sign | (mag == 0x7ff0000000000000ull ? 0x7c00u : 0x7e00u));
    if (mag == 0)
        return sign;
    uint64_t expfield = mag >> 52;
    uint64_t sig = mag & 0xfffffffffffffull;
    int e;
    if (expfield == 0) {
        e = -1074;
    } else {
        sig |= 0x10000000000000ull;
        e = (int)expfield - 1075;
    }
    return (uint16_t)(sign | half_from_scaled(sig, e));
}

float oracle_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expfield = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    float v;
    if (expfield == 0x1f) {
        v = frac ? NAN : INFINITY;
    } else if (expfield == 0) {
        v = ldexpf((float)frac, -24); /* exact */
    } else {
        v = ldexpf((float)(1024 + frac), expfield - 25); /* exact */
    }
    return sign ? -v : v;
}

void oracle_f32_to_f16_array(const float *x, uint16_t *out, int64_t count)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        out[i] = oracle_f32_to_f16(x[i]);
}

void oracle_f64_to_f16_array(const double *x, uint16_t *out, int64_t count)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i)
        out[i] = oracle_f64_to_f16(x[i]);
}

void oracle_f16_to_f32_array(const uint16_t *h, float *out, int64_t count)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = oracle_f16_to_f32(h[i]);
}

/* ------------------------------------------------------------------------ */
/* Row threshold (clip bound)                                               */
/* ------------------------------------------------------------------------ */

static int cmp_float_asc(const void *a, const void *b)
{
    float x = *(const float *)a, y = *(const float *)b;
    return (x > y) - (x < y);
}

/* The pct-th percentile of the k values |row[j]|, type-7 linear
 * interpolation between closest ranks, in binary64.  Returns the binary64
 * interpolated value; the threshold is its binary32 rounding.  For
 * pct == 100 this is the maximum (no clipping).  `scratch` holds k floats. */
double oracle_row_percentile(const float *row, int64_t k, double pct, float *scratch)
{
    for (int64_t j = 0; j < k; ++j)
        scratch[j] = fabsf(row[j]);
    if (pct == 100.0) {
        float mx = 0.0f;
        for (int64_t j = 0; j < k; ++j)
            if (scratch[j] > mx)
                mx = scratch[j];
        return (double)mx;
    }
    qsort(scratch, (size_t)k, sizeof(float), cmp_float_asc);
    double frac_of_range = pct / 100.0;
    double pos = frac_of_range * (double)(k - 1);
    double i_floor = floor(pos);
    int64_t i = (int64_t)i_floor;
    if (i >= k - 1)
        return (double)scratch[k - 1];
    double f = pos - i_floor;
    double lo = (double)scratch[i];
    double hi = (double)scratch[i + 1];
    double gap = hi - lo;
    double step = f * gap;
    return lo + step;
}

/* ------------------------------------------------------------------------ */
/* Quantizer                                                                */
/* ------------------------------------------------------------------------ */

/* Scale and codes of one row for the bound t (a2 and a3): S is the binary16
 * rounding of the binary32 quotient t / 127, and each code is the
 * round-half-even of the binary32 quotient w / S clamped to [-127, 127]
 * (LightSeq slide deck, slide "量化：裁剪+对称", symmetric formula with
 * n = 8 bits).  Returns S's bit pattern. */
static uint16_t quantize_row_with_bound(const float *row, int64_t k, float t, int8_t *qrow)
{
    float s32 = t / 127.0f;
    uint16_t s16 = oracle_f32_to_f16(s32);
    float s = oracle_f16_to_f32(s16);
    for (int64_t j = 0; j < k; ++j) {
        if (s == 0.0f) {
            qrow[j] = 0;
            continue;
        }
        float ratio = row[j] / s;       /* binary32 IEEE division */
        float rounded = rintf(ratio);  /* default mode: nearest, ties to even */
        if (rounded > 127.0f)
            rounded = 127.0f;
        if (rounded < -127.0f)
            rounded = -127.0f;
        qrow[j] = (int8_t)rounded;
    }
    return s16;
}

/* Quantize W[n][k] (row-major binary32) per output row, with the bound
 * taken from the row's data (its absmax, or the pct-th percentile of |w|).
 *   q       [n][k] int8 codes (out)
 *   scales  [n] binary16 bit patterns (out)
 *   thresh  [n] binary32 clip bound t (out, may be NULL)
 * Returns 0, or -1 for invalid arguments (non-finite input included). */
int oracle_quantize(const float *w, int64_t n, int64_t k, double pct,
                    int8_t *q, uint16_t *scales, float *thresh)
{
    if (n < 0 || k <= 0 || !(pct > 0.0 && pct <= 100.0))
        return -1;
    for (int64_t i = 0; i < n * k; ++i)
        if (!isfinite(w[i]))
            return -1;
    int bad = 0;
#pragma omp parallel
    {
        float *scratch = (float *)malloc((size_t)k * sizeof(float));
        if (!scratch) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < n; ++r) {
            if (!scratch)
                continue;
            const float *row = w + r * k;
            double t64 = oracle_row_percentile(row, k, pct, scratch);
            float t = (float)t64;
            scales[r] = quantize_row_with_bound(row, k, t, q + r * k);
            if (thresh)
                thresh[r] = t;
        }
        free(scratch);
    }
    return bad ? -1 : 0;
}

/* Outlier-aware quantization (dense int8 inliers plus a sparse list of
 * exact outliers).  Source: GOBO review (nubint.ai), section on the method:
 * weights are Gaussian apart from a small fraction of outliers (about
 * 0.1%), which are kept exactly in a side list while the rest is
 * quantized.  Reading: the outliers of row r are the elements with
 * |w| > t[r], the row's clip bound (the same bound as oracle_quantize with
 * the given percentile; pct = 100 has none).  They are stored in the row's
 * `cap` slots of ol_idx / ol_val in ascending column order (value exact in
 * binary32; unused slots: index -1, value 0) and their codes are 0; every
 * other code is the clipped quantizer's.  Rows whose scale is 0 keep no
 * outliers (all their codes are 0, as in oracle_quantize).  Returns 0, or
 * -1 for invalid arguments or a row with more than `cap` outliers. */
int oracle_quantize_outliers(const float *w, int64_t n, int64_t k, double pct, int8_t *q,
                             uint16_t *scales, int32_t *ol_idx, float *ol_val, int64_t cap)
{
    if (cap < 0)
        return -1;
    float *thresh = (float *)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    if (!thresh)
        return -1;
    int rc = oracle_quantize(w, n, k, pct, q, scales, thresh);
    int over = 0;
    for (int64_t r = 0; rc == 0 && r < n; ++r) {
        const float *row = w + r * k;
        int64_t used = 0;
        for (int64_t e = 0; e < cap; ++e) {
            ol_idx[r * cap + e] = -1;
            ol_val[r * cap + e] = 0.0f;
        }
        if (oracle_f16_to_f32(scales[r]) == 0.0f)
            continue;
        for (int64_t j = 0; j < k; ++j) {
            if (fabsf(row[j]) > thresh[r]) {
                if (used == cap) {
                    over = 1;
                    break;
                }
                ol_idx[r * cap + used] = (int32_t)j;
                ol_val[r * cap + used] = row[j];
                q[r * k + j] = 0;
                ++used;
            }
        }
    }
    free(thresh);
    return (rc != 0 || over) ? -1 : 0;
}

/* Slots per row that always hold a row's outliers: the elements above the
 * type-7 bound lie among the k - 1 - floor(pos) largest, pos = (pct/100)(k-1)
 * in binary64; none for pct = 100. */
int64_t oracle_outlier_capacity(int64_t k, double pct)
{
    if (pct == 100.0)
        return 0;
    double frac_of_range = pct / 100.0;
    double pos = frac_of_range * (double)(k - 1);
    int64_t i = (int64_t)floor(pos);
    return i >= k - 1 ? 0 : k - 1 - i;
}

/* Fixed-range clip: the bound of row r is given (bounds[r], finite and
 * >= 0, e.g. a range fixed during training) instead of being measured on
 * the row; the scale and codes then follow exactly as above.  Source:
 * LightSeq slide deck, slide "量化流程" (fixed range clip next to the
 * percentage clip).  Returns 0, or -1 for invalid arguments. */
int oracle_quantize_fixed(const float *w, int64_t n, int64_t k, const float *bounds,
                          int8_t *q, uint16_t *scales)
{
    if (n < 0 || k <= 0)
        return -1;
    for (int64_t i = 0; i < n * k; ++i)
        if (!isfinite(w[i]))
            return -1;
    for (int64_t r = 0; r < n; ++r)
        if (!isfinite(bounds[r]) || bounds[r] < 0.0f)
            return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        scales[r] = quantize_row_with_bound(w + r * k, k, bounds[r], q + r * k);
    return 0;
}

/* Asymmetric (zero-point) quantization of W[n][k], 8 bits stored as int8.
 * Source: LightSeq slide deck, slide "量化：裁剪+对称" (asymmetric case: the
 * range [min, max] is spread over the 2^n - 1 steps with scale S and a zero
 * point z, and a product of two such values expands into the code product
 * plus zero-point cross terms).  Per row:
 *   hi = max(0, max w), lo = min(0, min w)   (the range holds 0, so 0 is
 *                                             exactly representable)
 *   S  = binary16_RNE( binary32( binary32(hi - lo) / 255 ) )
 *   z  = clamp( round_half_even( binary32(-lo / S) ) - 128, -128, 127 )
 *   q  = clamp( round_half_even( binary32(w / S) ) + z, -128, 127 )
 *   (S == 0: z = 0 and q = 0)
 * so that w ~ S * (q - z), w = 0 maps to code z and lo to code -128.
 * Returns 0, or -1 for invalid arguments (non-finite input included). */
int oracle_quantize_asym(const float *w, int64_t n, int64_t k, int8_t *q, uint16_t *scales,
                         int8_t *zeros)
{
    if (n < 0 || k <= 0)
        return -1;
    for (int64_t i = 0; i < n * k; ++i)
        if (!isfinite(w[i]))
            return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        const float *row = w + r * k;
        int8_t *qrow = q + r * k;
        float hi = 0.0f, lo = 0.0f;
        for (int64_t j = 0; j < k; ++j) {
            if (row[j] > hi)
                hi = row[j];
            if (row[j] < lo)
                lo = row[j];
        }
        float range = hi - lo;
        float s32 = range / 255.0f;
        uint16_t s16 = oracle_f32_to_f16(s32);
        float s = oracle_f16_to_f32(s16);
        scales[r] = s16;
        if (s == 0.0f) {
            zeros[r] = 0;
            for (int64_t j = 0; j < k; ++j)
                qrow[j] = 0;
            continue;
        }
        float zf = rintf(-lo / s) - 128.0f;
        if (zf > 127.0f)
            zf = 127.0f;
        if (zf < -128.0f)
            zf = -128.0f;
        zeros[r] = (int8_t)zf;
        for (int64_t j = 0; j < k; ++j) {
            float c = rintf(row[j] / s) + zf;
            if (c > 127.0f)
                c = 127.0f;
            if (c < -128.0f)
                c = -128.0f;
            qrow[j] = (int8_t)c;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* W8A16 matmul reference                                                   */
/* ------------------------------------------------------------------------ */

/* One output: sum_k x[m][k] * ((q[n][k] - z[n]) * S[n]) in binary64 (z = 0
 * for the symmetric quantizer).  x holds binary16 bit patterns.  Every
 * product is exact in binary64 (11 x 9 x 11 significant bits); only the
 * K-term sum rounds. */
static double dot_one(const uint16_t *xrow, const int8_t *qrow, double z, double s, int64_t k)
{
    double acc = 0.0;
    for (int64_t j = 0; j < k; ++j) {
        double wdeq = ((double)qrow[j] - z) * s;
        double xv = (double)oracle_f16_to_f32(xrow[j]);
        acc += xv * wdeq;
    }
    return acc;
}

/* Full reference: ref[m][n] for X[m][k] (binary16 bits), Q[n][k], S[n]
 * (binary16 bits). */
void oracle_gemm(const uint16_t *x, const int8_t *q, const uint16_t *scales,
                 int64_t m, int64_t n, int64_t k, double *ref)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j)
            ref[i * n + j] = dot_one(x + i * k, q + j * k, 0.0,
                                     (double)oracle_f16_to_f32(scales[j]), k);
}

/* Sampled reference: out[c] = ref[mi[c]][ni[c]]. */
void oracle_gemm_sampled(const uint16_t *x, const int8_t *q, const uint16_t *scales,
                         int64_t k, const int64_t *mi, const int64_t *ni,
                         int64_t count, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < count; ++c)
        out[c] = dot_one(x + mi[c] * k, q + ni[c] * k, 0.0,
                         (double)oracle_f16_to_f32(scales[ni[c]]), k);
}

/* Outlier-aware matmul: the dense int8 part plus the exact outliers,
 * ref[m][n] = sum_k x[m][k] * (q[n][k] * S[n]) + sum_e x[m][idx[n][e]] * val[n][e]
 * over the used slots (idx >= 0), in binary64. */
static double outliers_one(const uint16_t *xrow, const int32_t *idx, const float *val, int64_t cap)
{
    double acc = 0.0;
    for (int64_t e = 0; e < cap; ++e) {
        if (idx[e] < 0)
            continue;
        double xv = (double)oracle_f16_to_f32(xrow[idx[e]]);
        acc += xv * (double)val[e];
    }
    return acc;
}

void oracle_gemm_outliers(const uint16_t *x, const int8_t *q, const uint16_t *scales,
                          const int32_t *ol_idx, const float *ol_val, int64_t cap,
                          int64_t m, int64_t n, int64_t k, double *ref)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            const double dense = dot_one(x + i * k, q + j * k, 0.0, (double)oracle_f16_to_f32(scales[j]), k);
            ref[i * n + j] = dense + outliers_one(x + i * k, ol_idx + j * cap, ol_val + j * cap, cap);
        }
}

void oracle_gemm_outliers_sampled(const uint16_t *x, const int8_t *q, const uint16_t *scales,
                                  const int32_t *ol_idx, const float *ol_val, int64_t cap, int64_t k,
                                  const int64_t *mi, const int64_t *ni, int64_t count, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < count; ++c) {
        const double dense = dot_one(x + mi[c] * k, q + ni[c] * k, 0.0,
                                     (double)oracle_f16_to_f32(scales[ni[c]]), k);
        out[c] = dense + outliers_one(x + mi[c] * k, ol_idx + ni[c] * cap, ol_val + ni[c] * cap, cap);
    }
}

/* Asymmetric weights: ref[m][n] = sum_k x[m][k] * ((q[n][k] - z[n]) * S[n]),
 * the dequantization S * (q - z) of the asymmetric slide. */
void oracle_gemm_asym(const uint16_t *x, const int8_t *q, const uint16_t *scales,
                      const int8_t *zeros, int64_t m, int64_t n, int64_t k, double *ref)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            const double zj = (double)zeros[j];
            ref[i * n + j] = dot_one(x + i * k, q + j * k, zj, (double)oracle_f16_to_f32(scales[j]), k);
        }
}

void oracle_gemm_asym_sampled(const uint16_t *x, const int8_t *q, const uint16_t *scales,
                              const int8_t *zeros, int64_t k, const int64_t *mi, const int64_t *ni,
                              int64_t count, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < count; ++c) {
        const double zc = (double)zeros[ni[c]];
        out[c] = dot_one(x + mi[c] * k, q + ni[c] * k, zc, (double)oracle_f16_to_f32(scales[ni[c]]), k);
    }
}

/* ------------------------------------------------------------------------ */
/* W8A8: activations quantized per row (per token) with the same symmetric  */
/* quantizer as the weights, so both operands are int8 codes with one scale */
/* per row.  The product of two symmetric quantized values is the product   */
/* of their codes times the two scales, with no zero-point cross terms      */
/* (LightSeq slide deck, slide "量化：裁剪+对称", symmetric case), which    */
/* makes the matmul an exact integer dot product scaled once at the end;    */
/* LightSeq's engine runs it as an int8 GEMM ("最高加速9倍！字節跳動開源8比特 */
/* 混合精度Transformer引擎（1）", section on quantized inference speed).     */
/*                                                                          */
/*   ref[m][n] = (sum_k qx[m][k] * q[n][k]) * (Sx[m] * S[n])                */
/*                                                                          */
/* The integer sum is exact in int64; Sx * S is exact in binary64 (two      */
/* 11-bit significands); the final product rounds once in binary64.         */

static double w8a8_one(const int8_t *xrow, const int8_t *qrow, double sx, double sw, int64_t k)
{
    int64_t acc = 0;
    for (int64_t j = 0; j < k; ++j)
        acc += (int64_t)xrow[j] * (int64_t)qrow[j];
    return (double)acc * (sx * sw);
}

/* Full reference for QX[m][k], SX[m] (binary16 bits), Q[n][k], S[n]
 * (binary16 bits). */
void oracle_w8a8_gemm(const int8_t *qx, const uint16_t *sx, const int8_t *q,
                      const uint16_t *scales, int64_t m, int64_t n, int64_t k, double *ref)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            const double sw = (double)oracle_f16_to_f32(scales[j]);
            ref[i * n + j] = w8a8_one(qx + i * k, q + j * k, (double)oracle_f16_to_f32(sx[i]), sw, k);
        }
}

/* Sampled reference: out[c] = ref[mi[c]][ni[c]]. */
void oracle_w8a8_gemm_sampled(const int8_t *qx, const uint16_t *sx, const int8_t *q,
                              const uint16_t *scales, int64_t k, const int64_t *mi,
                              const int64_t *ni, int64_t count, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < count; ++c)
        out[c] = w8a8_one(qx + mi[c] * k, q + ni[c] * k, (double)oracle_f16_to_f32(sx[mi[c]]),
                          (double)oracle_f16_to_f32(scales[ni[c]]), k);
}

/* Threads the OpenMP runtime will use for the parallel loops above. */
int oracle_num_threads(void)
{
    int nt = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#if defined(_OPENMP)
            nt = omp_get_num_threads();
#endif
        }
    }
    return nt;
}

/*
 * qw.h -- int8 weight-only (W8A16) Linear layers for AMD Instinct MI355X
 * (gfx950): a C ABI over hand-written HIP kernels.
 *
 * The method (restated from the pages, not quoted):
 *   - Symmetric 8-bit quantization maps a per-channel bound onto the
 *     largest code 2^(8-1)-1 = 127 with q = round(w / S); optional clipping
 *     of the bound by a percentage of the weight magnitudes.  Source: LightSeq
 *     slide deck "LightSeq：高性能NLP序列推理实践", slides "量化流程" and
 *     "量化：裁剪+对称".
 *   - Only Linear weights are quantized (per channel, stored int8 with an
 *     F16 scale); at compute time they are cast back to F16, scaled and
 *     multiplied with F16 activations; the weight is the right, 2-D operand.
 *     Source: "探索ChatGLM2在算能BM1684X上INT8量化部署" (elecfans),
 *     sections 2 (量化方案), 3 (TPU-MLIR实现) and 4 (后端性能提升原理).
 *
 * Conventions for every entry point:
 *   - Matrices are row-major and contiguous.  W / Q are [n][k] (torch
 *     Linear layout: n output channels, k input features, k contiguous),
 *     X is [m][k], Y is [m][n].  fp16 values travel as their IEEE binary16
 *     bit patterns (uint16_t).
 *   - Every pointer is a HIP device pointer (or managed memory visible to
 *     the device) owned by the caller; the library allocates no device
 *     memory and keeps no per-call state.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream),
 *     passed as `void *` so that this header needs no HIP include; the two
 *     have the same representation (hipStream_t is a pointer type).  Calls
 *     enqueue work on it and return without waiting; results are visible
 *     after the caller synchronizes the stream.
 *   - Arguments are checked on the host before anything is enqueued; on
 *     any error nothing is launched and no output byte is written.
 *   - Results are deterministic: every floating-point reduction runs in a
 *     fixed order.  The only atomics are integer additions into the
 *     percentile quantizer's LDS histogram, whose counts do not depend on
 *     the order of the additions; no global-memory atomics are used.
 *   - Not safe to call with overlapping input and output buffers
 *     (rejected with QW_ERROR_INVALID_VALUE when detected).
 */
#ifndef QW_H
#define QW_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define QW_API __attribute__((visibility("default")))
#else
#define QW_API
#endif

typedef enum qw_status {
    QW_SUCCESS = 0,
    QW_ERROR_INVALID_VALUE = 1, /* null pointer, negative size, k == 0, bad percentile, overlap */
    QW_ERROR_MISALIGNED = 2,    /* a pointer is not 16-byte aligned */
    QW_ERROR_UNSUPPORTED = 3,   /* k % 16 != 0, or a size beyond the documented maximum */
    QW_ERROR_LAUNCH = 4         /* the HIP runtime rejected a launch (no device, bad stream, ...) */
} qw_status;

/* Largest row length the quantizer accepts (a row is held in registers). */
#define QW_QUANTIZE_MAX_K 65536
/* Longest reduction qw_w8a8_gemm accepts: the int32 accumulator holds
 * k * 127 * 127 without overflow for k <= 2^17. */
#define QW_W8A8_MAX_K 131072
/* Longest reduction the LDS-tiled MFMA kernel (QW_PATH_MFMA) takes: its
 * 32-bit in-tile offsets stay below 2^31 for k <= 2^23.  qw_w8a16_gemm runs
 * longer rows on the skinny kernel. */
#define QW_MFMA_MAX_K 8388608

/*
 * qw_quantize_weights -- per-output-channel symmetric int8 quantization.
 *
 * Source: LightSeq slide deck, slides "量化流程" (fixed range clip vs
 * percentage clip) and "量化：裁剪+对称" (bound -> 2^(n-1)-1, q = round(w/S));
 * ChatGLM2/BM1684X page, section 2 (per-channel weight-only int8) and
 * section 3 (F16 scale).
 *
 * For every row r of W[n][k] (fp32):
 *   t[r]  = largest |W[r][j]| if clip_percentile == 100, otherwise the
 *           clip_percentile-th percentile of |W[r][:]| with linear
 *           interpolation between closest ranks (a = |row| sorted
 *           ascending, pos = (clip_percentile / 100) * (k - 1) in binary64,
 *           i = floor(pos), t = a[i] + (pos - i) * (a[i+1] - a[i]) in
 *           binary64 without fused multiply-add, then rounded to binary32;
 *           i >= k - 1 gives a[k-1]);
 *   S[r]  = binary16( binary32( t[r] / 127 ) ), both roundings to nearest
 *           even, true IEEE division;
 *   q[r][j] = 0 if S[r] == 0, else clamp( round_half_even( binary32(
 *           W[r][j] / S[r] ) ), -127, 127 ) -- the quotient divides by the
 *           stored binary16 scale.  -128 is never produced.
 *
 *   w                fp32 [n][k], read only, finite values (non-finite input
 *                    gives unspecified codes)
 *   n                rows (output channels), 0 <= n <= INT32_MAX; n == 0 is a no-op
 *   k                row length, 16 <= k <= QW_QUANTIZE_MAX_K, k % 16 == 0
 *   clip_percentile  in (0, 100]; 100 means no clipping (absmax).  binary64,
 *                    so that e.g. 99.99 is not first rounded to binary32
 *   q                int8 [n][k] codes (written)
 *   scales           binary16 bits [n] (written)
 *   stream           hipStream_t
 *
 * Errors: QW_ERROR_INVALID_VALUE (null pointer with n > 0, n < 0, k <= 0,
 * clip_percentile NaN or outside (0, 100], q/scales overlapping w or each
 * other), QW_ERROR_UNSUPPORTED (k % 16 != 0, k > QW_QUANTIZE_MAX_K,
 * n > INT32_MAX), QW_ERROR_MISALIGNED (w, q or scales not 16-byte aligned),
 * QW_ERROR_LAUNCH.  Bit-exact by contract: the same inputs give the same
 * bytes on every call.
 */
QW_API qw_status qw_quantize_weights(const float *w, int64_t n, int64_t k,
                                     double clip_percentile, int8_t *q,
                                     uint16_t *scales, void *stream);

/*
 * qw_quantize_weights_f16 -- qw_quantize_weights for fp16 weights (the dtype
 * the ChatGLM2/BM1684X page's model ships in, section 1), and the per-token
 * quantizer of fp16 activations for the W8A8 product below.
 *
 * Every weight is first widened exactly to binary32; everything else is
 * qw_quantize_weights's contract word for word, so the codes and scales
 * equal those of qw_quantize_weights on the widened matrix.
 *
 *   w   fp16 bits [n][k], read only
 *   (other arguments and errors as qw_quantize_weights; the overlap checks
 *   use 2 bytes per input weight)
 */
QW_API qw_status qw_quantize_weights_f16(const uint16_t *w, int64_t n, int64_t k,
                                         double clip_percentile, int8_t *q,
                                         uint16_t *scales, void *stream);

/*
 * qw_quantize_weights_fixed_range -- the quantizer with each row's clip
 * bound given instead of measured (fixed-range clip).
 *
 * Source: LightSeq slide deck ("LightSeq：高性能NLP序列推理实践"), slide
 * 量化流程: a fixed range clip beside the percentage clip, both followed by
 * the symmetric quantization of slide 量化：裁剪+对称.  The bound of row r
 * is bounds[r] (for example a range fixed during quantization-aware
 * training); scale and codes then follow qw_quantize_weights exactly:
 *
 *   S[r] = binary16_RNE( binary32(bounds[r] / 127) )
 *   q[r][c] = clamp( round_half_even( binary32(w[r][c] / S[r]) ), -127, 127 )
 *   (q = 0 when S[r] == 0)
 *
 *   w       fp32 [n][k], read only
 *   bounds  fp32 [n], read only; each finite and >= 0 (other values give
 *           unspecified codes and scales; they are not checked on the host)
 *   q, scales, n, k, stream as qw_quantize_weights
 *
 * Errors: as qw_quantize_weights (no percentile argument), plus
 * QW_ERROR_INVALID_VALUE for a null bounds pointer or q or scales
 * overlapping bounds, and QW_ERROR_MISALIGNED for a misaligned bounds.
 */
QW_API qw_status qw_quantize_weights_fixed_range(const float *w, int64_t n, int64_t k,
                                                 const float *bounds, int8_t *q,
                                                 uint16_t *scales, void *stream);

/*
 * qw_outlier_capacity -- side-list slots per row that always hold the
 * outliers of qw_quantize_weights_outliers for this row length and clip
 * percentile: k - 1 - floor(pos), pos = (clip_percentile / 100) * (k - 1) in
 * binary64 (the elements above the type-7 bound are among the k - 1 - i
 * largest); 0 for clip_percentile = 100.  Returns -1 for k <= 0 or a
 * percentile outside (0, 100].
 */
QW_API int64_t qw_outlier_capacity(int64_t k, double clip_percentile);

/*
 * qw_quantize_weights_outliers -- outlier-aware quantization: dense int8
 * codes for the inliers plus an exact side list of the outliers.
 *
 * Source: GOBO review (nubint.ai), method section: Transformer weights are
 * Gaussian apart from a small fraction of outliers (about 0.1%), which are
 * kept at full precision in a side list while the rest is quantized.  The
 * outliers of row r are the elements with |w| > t[r], the clip bound of
 * qw_quantize_weights with the same clip_percentile; the scale and the
 * other codes are exactly qw_quantize_weights's, the outliers' codes are 0.
 * Rows whose scale is 0 keep no outliers (their codes are all 0).
 *
 *   w, n, k, clip_percentile, q, scales, stream as qw_quantize_weights
 *   ol_idx  int32 [n][cap] (written): the row's outlier columns in
 *           ascending order, then -1 in the unused slots
 *   ol_val  fp32 [n][cap] (written): the outliers' values, exact; 0 in the
 *           unused slots
 *   cap     slots per row, qw_outlier_capacity(k, clip_percentile) <= cap
 *           <= k (cap == 0 is allowed when the capacity is 0)
 *
 * Errors: as qw_quantize_weights, plus QW_ERROR_INVALID_VALUE for cap below
 * the capacity or above k, null side-list pointers, or side lists
 * overlapping w, q, scales or each other, and QW_ERROR_MISALIGNED for
 * misaligned side lists.
 */
QW_API qw_status qw_quantize_weights_outliers(const float *w, int64_t n, int64_t k,
                                              double clip_percentile, int8_t *q,
                                              uint16_t *scales, int32_t *ol_idx, float *ol_val,
                                              int64_t cap, void *stream);

/*
 * qw_w8a16_gemm_outliers -- W8A16 plus the exact outlier side lists:
 *
 *   Y[i][c] = binary16_RNE( S[c] * sum_j X[i][j] * q[c][j]
 *                           + sum_e X[i][ol_idx[c][e]] * ol_val[c][e] )
 *
 * over the used slots, in fp32 (the GOBO reading above: the dense int8
 * part plus the full-precision outliers).  The GEMV and skinny kernels add
 * the side list in their epilogues; the MFMA kernel adds it (in units of
 * S[c], value / S[c] in binary32) to its accumulators after the main loop,
 * for up to 4 slots per row (wider lists run on the skinny kernel, and
 * QW_PATH_MFMA with more than 4 slots is QW_ERROR_UNSUPPORTED).  Accuracy
 * contract as qw_w8a16_gemm.
 *
 *   ol_idx, ol_val, cap  as written by qw_quantize_weights_outliers: used
 *           slots first, columns ascending and < k (columns outside [0, k)
 *           end the row's list; entries out of order may be skipped by the
 *           MFMA kernel); rows with S[c] == 0 must have no used slots
 *   (other arguments as qw_w8a16_gemm; cap == 0 is the plain GEMM)
 *
 * Errors: as qw_w8a16_gemm, plus QW_ERROR_INVALID_VALUE for cap < 0 or
 * cap > k, null side lists with cap > 0, or y overlapping them, and
 * QW_ERROR_MISALIGNED for misaligned side lists.
 * qw_w8a16_gemm_outliers_path forces the kernel as qw_w8a16_gemm_path does.
 */
QW_API qw_status qw_w8a16_gemm_outliers(const uint16_t *x, const int8_t *q,
                                        const uint16_t *scales, const int32_t *ol_idx,
                                        const float *ol_val, int64_t cap, uint16_t *y,
                                        int64_t m, int64_t n, int64_t k, void *stream);
QW_API qw_status qw_w8a16_gemm_outliers_path(const uint16_t *x, const int8_t *q,
                                             const uint16_t *scales, const int32_t *ol_idx,
                                             const float *ol_val, int64_t cap, uint16_t *y,
                                             int64_t m, int64_t n, int64_t k, int path,
                                             void *stream);

/*
 * qw_quantize_weights_asym -- asymmetric (zero-point) per-row int8
 * quantization.
 *
 * Source: LightSeq slide deck ("LightSeq：高性能NLP序列推理实践"), slide
 * 量化：裁剪+对称, asymmetric case: the value range is spread over the
 * 2^n - 1 steps with a scale S and a zero point z, and W ~ S * (q - z).
 * Per row r, with the range widened to hold 0 so that 0 is exact:
 *
 *   hi = max(0, max_c w[r][c]),  lo = min(0, min_c w[r][c])
 *   S[r] = binary16_RNE( binary32( binary32(hi - lo) / 255 ) )
 *   z[r] = clamp( round_half_even( binary32(-lo / S[r]) ) - 128, -128, 127 )
 *   q[r][c] = clamp( round_half_even( binary32(w[r][c] / S[r]) ) + z[r], -128, 127 )
 *   (S[r] == 0: z[r] = 0 and q[r][:] = 0)
 *
 * so w = 0 maps to code z[r] and the row minimum (when negative) to -128.
 *
 *   w       fp32 [n][k], read only
 *   q       int8 [n][k] (written)
 *   scales  fp16 bits [n] (written)
 *   zeros   int8 [n] zero points (written)
 *   n, k, stream as qw_quantize_weights
 *
 * Errors: as qw_quantize_weights (no percentile argument), plus
 * QW_ERROR_INVALID_VALUE for a null zeros or zeros overlapping w, q or
 * scales, and QW_ERROR_MISALIGNED for a misaligned zeros.
 */
QW_API qw_status qw_quantize_weights_asym(const float *w, int64_t n, int64_t k, int8_t *q,
                                          uint16_t *scales, int8_t *zeros, void *stream);

/*
 * qw_w8a16_gemm -- Y = X * dequant(Q)^T with per-channel fp16 scales.
 *
 * Source: ChatGLM2/BM1684X page, section 4 (后端性能提升原理): load, cast
 * int8 -> F16, multiply by the scale (dequantize), matrix multiply with the
 * input activation, store; section 3: the quantized weight is the right
 * operand of the MatMul.
 *
 *   Y[i][c] = binary16_RNE( S[c] * sum_j X[i][j] * q[c][j] )
 *
 * The int8 -> fp16 cast is exact; products are formed exactly and summed in
 * binary32 (fp32 accumulation); the per-channel scale is applied to the
 * fp32 sum (algebraically the same as scaling each weight first, with less
 * rounding), and the MFMA kernels round that product to binary16 in one
 * fused step (a zero product is written as +0).  The decode GEMV (one or
 * two activation rows, k <= 8192) sums each 16-code chunk as
 * sum x (1152 + q) - sum x 1152 (the cast's bias subtracted once per chunk
 * instead of per code), both chains formed exactly in the same order, so a
 * row of zero codes still sums to +0 and integer inputs whose partial sums
 * stay below 2^24 are still exact.  Accuracy contract:
 * max |Y - exact| <= 2e-3 * max|exact| + 1e-3.
 *
 *   x       fp16 bits [m][k]
 *   q       int8 [n][k] codes (as written by qw_quantize_weights)
 *   scales  fp16 bits [n]
 *   y       fp16 bits [m][n] (written)
 *   m       rows of X, 0 <= m <= INT32_MAX; m == 0 is a no-op
 *   n       output channels, 0 <= n <= INT32_MAX; n == 0 is a no-op
 *   k       reduction length, k >= 16, k % 16 == 0, k <= INT32_MAX
 *   stream  hipStream_t
 *
 * The kernel is chosen from m, n and k: a bandwidth-bound VALU GEMV for
 * decode (m <= 2), a skinny MFMA kernel on register-dequantized weights for
 * a few activation rows (m <= 16, and beyond while it needs at most 8
 * passes over the weights, one per 16 or 32 rows, and the passes after the
 * first read at most 128 MiB) and for k > QW_MFMA_MAX_K, and the LDS-tiled
 * MFMA GEMM (tile shape picked from the grid it fills) otherwise.
 *
 * Errors: QW_ERROR_INVALID_VALUE (null pointer with m, n > 0, negative
 * size, k <= 0, y overlapping x, q or scales), QW_ERROR_UNSUPPORTED
 * (k % 16 != 0, a size beyond INT32_MAX), QW_ERROR_MISALIGNED,
 * QW_ERROR_LAUNCH.
 */
QW_API qw_status qw_w8a16_gemm(const uint16_t *x, const int8_t *q,
                               const uint16_t *scales, uint16_t *y, int64_t m,
                               int64_t n, int64_t k, void *stream);

/* Kernel selection for qw_w8a16_gemm_path. */
typedef enum qw_gemm_path {
    QW_PATH_AUTO = 0,   /* what qw_w8a16_gemm does */
    QW_PATH_GEMV = 1,   /* VALU dot products, weights streamed once (m <= 8; X in registers for m <= 2) */
    QW_PATH_MFMA = 2,   /* MFMA tiled GEMM, int8 tiles dequantized into LDS */
    QW_PATH_SKINNY = 3  /* MFMA on weights dequantized in registers, 16 (or 32) activation rows per pass */
} qw_gemm_path;

/*
 * qw_w8a16_gemm_path -- qw_w8a16_gemm with the kernel forced, for parity
 * tests of each path and for measuring the decode/prefill crossover.  Same
 * arguments, result contract and errors as qw_w8a16_gemm, plus
 * QW_ERROR_INVALID_VALUE for an unknown path and QW_ERROR_UNSUPPORTED when
 * a kernel is forced outside its limits: QW_PATH_GEMV with m > 8 or
 * m * ceil(k / 1024) > 32, QW_PATH_MFMA with k > QW_MFMA_MAX_K,
 * QW_PATH_SKINNY with m > 16 * 65535.
 */
QW_API qw_status qw_w8a16_gemm_path(const uint16_t *x, const int8_t *q,
                                    const uint16_t *scales, uint16_t *y,
                                    int64_t m, int64_t n, int64_t k, int path,
                                    void *stream);

/*
 * qw_w8a16_gemm_asym -- W8A16 with asymmetric weights (as written by
 * qw_quantize_weights_asym):
 *
 *   Y[i][c] = binary16_RNE( S[c] * sum_j X[i][j] * (q[c][j] - z[c]) )
 *
 * the dequantization S * (q - z) of the asymmetric slide (LightSeq deck,
 * 量化：裁剪+对称).  q - z is formed exactly in fp16 by the int8 cast (it
 * lies in [-255, 255]); products are exact in fp32 and summed in fp32, as
 * in qw_w8a16_gemm, with the same kernels, kernel choice and accuracy
 * contract.  zeros: int8 [n], 16-byte aligned.  Errors: as qw_w8a16_gemm,
 * plus QW_ERROR_INVALID_VALUE for a null zeros (m, n > 0) or y overlapping
 * zeros, and QW_ERROR_MISALIGNED for a misaligned zeros.
 * qw_w8a16_gemm_asym_path forces the kernel as qw_w8a16_gemm_path does.
 */
QW_API qw_status qw_w8a16_gemm_asym(const uint16_t *x, const int8_t *q, const uint16_t *scales,
                                    const int8_t *zeros, uint16_t *y, int64_t m, int64_t n,
                                    int64_t k, void *stream);
QW_API qw_status qw_w8a16_gemm_asym_path(const uint16_t *x, const int8_t *q,
                                         const uint16_t *scales, const int8_t *zeros,
                                         uint16_t *y, int64_t m, int64_t n, int64_t k, int path,
                                         void *stream);

/*
 * qw_w8a16_gemm_auto_path -- the QW_PATH_* kernel qw_w8a16_gemm would run
 * for this shape (for benchmarks and logs).  Returns -1 for shapes the GEMM
 * rejects (m, n < 0, k <= 0, k % 16 != 0).
 */
QW_API int qw_w8a16_gemm_auto_path(int64_t m, int64_t n, int64_t k);

/*
 * qw_w8a16_gemm_mfma_tile -- the output tile QW_PATH_MFMA uses for this
 * shape on the current HIP device, encoded BN * 1000 + BM (BN output
 * channels x BM activation rows per workgroup: 256256, 256128, 256064,
 * 128128 or 128064), for benchmarks, logs and tests.  256256 is the
 * 8-wave ping-pong kernel (one workgroup per CU, two wave groups that take
 * turns at the matrix cores), chosen where its grid covers at least half
 * the device's CUs, rounding m up to 256 rows adds at most 10% over
 * rounding it to 64, and k <= QW_PINGPONG_MAX_K (calls with outlier side
 * lists keep the 4-wave tiles unless the tile is forced).  Otherwise the choice
 * depends on the device's CU count and the 4-wave kernels' occupancy
 * (queried once per device): the largest tile whose grid fills three
 * quarters of the workgroups the chip holds at once, else 128 x 64.
 * Returns -1 for shapes the GEMM rejects (m, n <= 0, k <= 0, k % 16 != 0,
 * a size beyond INT32_MAX) or when no HIP device is current.
 */
QW_API int qw_w8a16_gemm_mfma_tile(int64_t m, int64_t n, int64_t k);

/* Longest reduction the 256 x 256 ping-pong tile takes (its 256-row
 * activation tile spans 256 * k * 2 bytes of one 32-bit buffer range). */
#define QW_PINGPONG_MAX_K 4194304

/*
 * qw_w8a16_gemm_tile -- the MFMA GEMM (QW_PATH_MFMA) with a given output
 * tile, for tests, benchmarks and callers that pin the kernel per shape.
 * Computes what qw_w8a16_gemm (zeros and ol_idx null), qw_w8a16_gemm_asym
 * (zeros non-null) or qw_w8a16_gemm_outliers (cap > 0) computes, with the
 * same contracts.
 *
 *   x, q, scales, y, m, n, k, stream   as qw_w8a16_gemm
 *   zeros   int8 [n] zero points, or null for symmetric codes
 *   ol_idx, ol_val, cap   side lists as qw_w8a16_gemm_outliers (cap 0:
 *           none, and then both pointers may be null)
 *   tile    256256, 256128, 256064, 128128 or 128064 (BN * 1000 + BM)
 *
 * Errors: as the matching entry point with QW_PATH_MFMA forced, plus
 * QW_ERROR_INVALID_VALUE for any other tile, or for zeros with cap > 0
 * (side lists belong to symmetric codes), and QW_ERROR_UNSUPPORTED for
 * tile 256256 with k > QW_PINGPONG_MAX_K.
 */
QW_API qw_status qw_w8a16_gemm_tile(const uint16_t *x, const int8_t *q, const uint16_t *scales,
                                    const int8_t *zeros, const int32_t *ol_idx, const float *ol_val,
                                    int64_t cap, uint16_t *y, int64_t m, int64_t n, int64_t k, int tile,
                                    void *stream);

/*
 * qw_w8a16_gemm_tune -- per-shape autotuning of the W8A16 kernel choice.
 *
 * Source: LightSeq article ("最高加速9倍！字節跳動開源8比特混合精度
 * Transformer引擎（1）", section on quantized inference speed): int8 GEMMs
 * were slower than fp16 at some shapes until each shape was tuned
 * automatically; LightSeq deck, TVM part: per-shape parameter search with
 * the token count padded to a multiple of 8.  This call runs every
 * candidate (the GEMV when m and k allow it, the skinny kernel, and the
 * MFMA kernel with each of its five tiles, the ping-pong tile only for
 * k <= QW_PINGPONG_MAX_K) on the given buffers and
 * stream, times each with HIP events (two untimed rounds, then seven rounds
 * of one launch per candidate; the median decides), and records the
 * fastest for the bucket (current device, n, k,
 * m rounded up to a multiple of 8).  Every later automatic kernel choice
 * for that bucket (qw_w8a16_gemm, its asymmetric and outlier variants,
 * qw_w8a16_gemm_auto_path, qw_w8a16_gemm_mfma_tile) uses the record.
 *
 * Arguments, layout and errors as qw_w8a16_gemm; y holds the winner's
 * result.  The call synchronizes with `stream` and is meant for set-up, not
 * for the steady state.  Records are process-wide host state (a map under a
 * mutex); QW_ERROR_LAUNCH if a launch or an event call fails.
 *
 * qw_w8a16_gemm_tuned_choice -- the record for the bucket of (m, n, k) on
 * the current device: path * 1000000 + tile (tile = BN * 1000 + BM for
 * QW_PATH_MFMA, 0 otherwise), or -1 if none (or bad shape).
 * qw_w8a16_gemm_tune_reset -- forget every record (W8A16 and W8A8).
 */
QW_API qw_status qw_w8a16_gemm_tune(const uint16_t *x, const int8_t *q, const uint16_t *scales,
                                    uint16_t *y, int64_t m, int64_t n, int64_t k, void *stream);
QW_API int qw_w8a16_gemm_tuned_choice(int64_t m, int64_t n, int64_t k);
QW_API void qw_w8a16_gemm_tune_reset(void);

/*
 * qw_w8a8_gemm -- Y = (QX * Q^T) scaled by Sx[i] * S[c]: both operands int8
 * with one fp16 scale per row (W8A8).
 *
 * Source: LightSeq slide deck ("LightSeq：高性能NLP序列推理实践"), slide
 * 量化：裁剪+对称: the product of two symmetrically quantized values is the
 * product of their codes times both scales, with no zero-point cross terms,
 * so the matmul runs on int8 codes and the scales are applied once at the
 * end; LightSeq's article ("最高加速9倍！字節跳動開源8比特混合精度
 * Transformer引擎（1）", section on quantized inference speed) runs
 * Transformer GEMMs this way as int8 GEMMs.  The activation codes and
 * scales come from quantizing each activation row (token) with the
 * weights' quantizer, qw_quantize_weights_f16 with clip_percentile 100.
 *
 *   acc[i][c] = sum_j QX[i][j] * Q[c][j]       exact, int32
 *   Y[i][c]   = binary16_RNE( float(acc) * (S[c] * Sx[i]) )
 *
 * float(acc) rounds to binary32 only when |acc| >= 2^24; S[c] * Sx[i] is
 * exact in binary32.  The MFMA kernel rounds the product to binary16 in
 * one fused step (v_fma_mix), the skinny kernel through binary32; a zero
 * product may be written as +0 whatever the sign of acc.  Accuracy
 * contract: |Y - exact| <= 2^-10 |exact| + 2^-24 element-wise (one
 * binary16 rounding plus at most two binary32 roundings); bit-exact when
 * |acc| < 2^24 and the scales are powers of two.
 *
 *   qx      int8 [m][k] activation codes
 *   sx      fp16 bits [m], one scale per activation row
 *   q       int8 [n][k] weight codes (as written by qw_quantize_weights)
 *   scales  fp16 bits [n]
 *   y       fp16 bits [m][n] (written)
 *   m, n    as qw_w8a16_gemm (m == 0 or n == 0 is a no-op)
 *   k       16 <= k <= QW_W8A8_MAX_K, k % 16 == 0
 *   stream  hipStream_t
 *
 * Kernels: for a few activation rows (where qw_w8a16_gemm would not pick
 * its MFMA GEMM) the skinny kernel on v_mfma_i32_16x16x64_i8, else the
 * LDS-tiled MFMA GEMM on v_mfma_i32_32x32x32_i8, tile shape picked as for
 * qw_w8a16_gemm's MFMA path.  qw_w8a8_gemm_path forces QW_PATH_SKINNY or
 * QW_PATH_MFMA (QW_PATH_GEMV is QW_ERROR_INVALID_VALUE).  All pointers
 * 16-byte aligned.
 *
 * Errors: QW_ERROR_INVALID_VALUE (null pointer with m, n > 0, negative
 * size, k <= 0, y overlapping qx, sx, q or scales), QW_ERROR_UNSUPPORTED
 * (k % 16 != 0, k > QW_W8A8_MAX_K, m or n beyond INT32_MAX),
 * QW_ERROR_MISALIGNED, QW_ERROR_LAUNCH.
 */
QW_API qw_status qw_w8a8_gemm(const int8_t *qx, const uint16_t *sx, const int8_t *q,
                              const uint16_t *scales, uint16_t *y, int64_t m, int64_t n,
                              int64_t k, void *stream);
QW_API qw_status qw_w8a8_gemm_path(const int8_t *qx, const uint16_t *sx, const int8_t *q,
                                   const uint16_t *scales, uint16_t *y, int64_t m, int64_t n,
                                   int64_t k, int path, void *stream);

/*
 * qw_w8a8_gemm_auto_path -- the kernel qw_w8a8_gemm runs for this shape:
 * QW_PATH_SKINNY or QW_PATH_MFMA (a W8A8 tuning record for the shape's
 * bucket, else the shape rule of qw_w8a16_gemm without the GEMV); -1 for a
 * shape qw_w8a8_gemm rejects.
 */
QW_API int qw_w8a8_gemm_auto_path(int64_t m, int64_t n, int64_t k);

/*
 * qw_w8a8_gemm_tune -- per-shape autotuning of the W8A8 kernel choice, as
 * qw_w8a16_gemm_tune (same source passages, timing and bucket) over the
 * int8 kernels: the skinny kernel and the MFMA kernel with each of its
 * four tiles (256256, 256128, 256064, 128064).  The W8A8 records are kept apart
 * from the W8A16 ones; qw_w8a8_gemm, qw_w8a8_gemm_auto_path and
 * qw_w8a8_gemm_mfma_tile use them.  Arguments, layout and errors as
 * qw_w8a8_gemm; y holds the winner's result; the call synchronizes with
 * `stream`.
 *
 * qw_w8a8_gemm_tuned_choice -- the W8A8 record for the bucket of (m, n, k)
 * on the current device (encoding as qw_w8a16_gemm_tuned_choice), or -1.
 */
QW_API qw_status qw_w8a8_gemm_tune(const int8_t *qx, const uint16_t *sx, const int8_t *q,
                                   const uint16_t *scales, uint16_t *y, int64_t m, int64_t n,
                                   int64_t k, void *stream);
QW_API int qw_w8a8_gemm_tuned_choice(int64_t m, int64_t n, int64_t k);

/*
 * qw_w8a8_gemm_mfma_tile -- the output tile qw_w8a8_gemm uses for this
 * shape on the current HIP device (same encoding and rules as
 * qw_w8a16_gemm_mfma_tile, the ping-pong tile 256256 included, with the
 * W8A8 kernels' occupancy: 256256, 256128, 256064 or 128064; 128 x 128 is
 * not used).  Returns -1 for shapes qw_w8a8_gemm rejects or when no HIP
 * device is current.
 */
QW_API int qw_w8a8_gemm_mfma_tile(int64_t m, int64_t n, int64_t k);

/*
 * qw_w8a8_gemm_tile -- the W8A8 MFMA GEMM with a given output tile
 * (256256: the 8-wave ping-pong kernel, 256128, 256064 or 128064; BN * 1000
 * + BM), for tests, benchmarks and callers that pin the kernel per shape.
 * Arguments, result and errors as qw_w8a8_gemm, plus QW_ERROR_INVALID_VALUE
 * for any other tile.
 */
QW_API qw_status qw_w8a8_gemm_tile(const int8_t *qx, const uint16_t *sx, const int8_t *q,
                                   const uint16_t *scales, uint16_t *y, int64_t m, int64_t n, int64_t k,
                                   int tile, void *stream);

/*
 * Measurement aids.  Neither is part of the method; they put the GEMM
 * figures in context on the machine at hand.
 *
 * qw_probe_stream_read -- enqueue one plain streaming read of
 * floor(bytes / 1024) KiB starting at p (16-byte nontemporal loads, one
 * contiguous KiB per wave instruction, as the decode GEMV loads its
 * weights).  Its rate on a cold buffer is the practical read ceiling the
 * GEMV is compared with.  sink: one uint32 of device memory, written only
 * if a wave's folded bytes equal `magic` (pass any value; the write only
 * keeps the loads alive).  Errors: QW_ERROR_INVALID_VALUE (null p or sink
 * with bytes >= 1024, bytes < 0), QW_ERROR_MISALIGNED (p not 16-byte
 * aligned), QW_ERROR_LAUNCH.
 *
 * qw_probe_shader_clock -- enqueue one wave that spins for 20 us of the
 * 100 MHz constant clock and writes out[0] = shader-clock ticks elapsed
 * (s_memtime) and out[1] = constant-clock ticks elapsed (s_memrealtime);
 * the clock in MHz is 100 * out[0] / out[1].  Enqueued right after a timed
 * loop it reads the clock the loop left the chip at.  out: two uint64 of
 * device memory, 8-byte aligned.  Errors: QW_ERROR_INVALID_VALUE (null
 * out), QW_ERROR_MISALIGNED, QW_ERROR_LAUNCH.
 */
QW_API qw_status qw_probe_stream_read(const void *p, int64_t bytes, uint32_t magic, uint32_t *sink,
                                      void *stream);
QW_API qw_status qw_probe_shader_clock(uint64_t *out, void *stream);

/* A static, human-readable name for a status code (never NULL). */
QW_API const char *qw_status_string(qw_status status);

/* Library ABI version: major * 10000 + minor * 100 + patch. */
QW_API int qw_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QW_H */

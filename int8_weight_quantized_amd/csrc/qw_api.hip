// qw_api.hip -- the C ABI of libqw: argument checks, kernel selection and
// launch on the caller's stream.  No device memory is allocated here or in
// any kernel launcher; every check runs on the host before anything is
// enqueued, so a rejected call launches nothing and writes nothing.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "qw.h"
#include "qw_internal.h"

namespace qw {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];
} // namespace

int device_cu_count()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return 256;
    int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0)
        return cached;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    g_cu_count[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// Kernel choice by shape.  Decode (one or two activation rows): the VALU
// GEMV streams the weights once with the fewest instructions per byte.  A
// few rows: the skinny MFMA kernel keeps the weight stream at full rate
// while the VALU dot products would grow with m.  Prefill: the LDS-tiled
// MFMA GEMM, whose weight tiles are reused across activation rows.
//
// The skinny kernel takes 16 (or 32) activation rows per pass over the
// weights.  Passes beyond the first read the weights again, mostly from
// cache: the first few are nearly free on a small weight (they fill CUs
// the first leaves idle), later ones cost about 0.16-0.2 us per MB plus a
// fixed share; the MFMA kernel at these m costs about the same for any m
// (a few hundred tiles, each a long k loop).  In the crossover sweep over
// m at (k, n) = (4096, 27392), (4096, 4608) and (1024, 4096), timed
// round-robin, the skinny kernel is the faster one while it needs at most
// 8 passes and its extra passes read at most 128 MiB: up to 32 rows at
// (4096, 27392) and 128 at the two narrower weights.  The int8 kernels
// (W8A8) cross over at the same points, so they share the rule.
constexpr int64_t kSkinnyMaxPasses = 8;
constexpr int64_t kSkinnyExtraPassBytes = int64_t(128) << 20;

bool skinny_preferred(int64_t m, int64_t n, int64_t k)
{
    if (m <= 16)
        return true;
    const int64_t rows = skinny_rows_per_pass(m, k);
    const int64_t passes = (m + rows - 1) / rows;
    return passes <= kSkinnyMaxPasses && (passes - 1) * n * k <= kSkinnyExtraPassBytes;
}

int auto_path(int64_t m, int64_t n, int64_t k)
{
    if (m <= 2 && gemv_supported(m, k))
        return QW_PATH_GEMV;
    // rows longer than the MFMA kernel takes also go to the skinny kernel
    if (k > kMfmaMaxK || skinny_preferred(m, n, k))
        return QW_PATH_SKINNY;
    return QW_PATH_MFMA;
}

int auto_path_w8a8(int64_t m, int64_t n, int64_t k)
{
    return skinny_preferred(m, n, k) ? QW_PATH_SKINNY : QW_PATH_MFMA;
}

} // namespace qw

namespace {

constexpr int64_t kMaxDim = 0x7fffffff;

bool misaligned(const void *p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) != 0;
}

// Half-open byte ranges [a, a + na) and [b, b + nb) intersect.
bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb)
{
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + nb && pb < pa + na;
}

qw_status launch_status(hipError_t e)
{
    return e == hipSuccess ? QW_SUCCESS : QW_ERROR_LAUNCH;
}

qw_status check_gemm_args(const uint16_t *x, const int8_t *q, const uint16_t *scales, uint16_t *y,
                          int64_t m, int64_t n, int64_t k, bool &noop)
{
    noop = false;
    if (m < 0 || n < 0 || k <= 0)
        return QW_ERROR_INVALID_VALUE;
    if (m == 0 || n == 0) {
        noop = true;
        return QW_SUCCESS;
    }
    if (!x || !q || !scales || !y)
        return QW_ERROR_INVALID_VALUE;
    if (k % 16 != 0 || m > kMaxDim || n > kMaxDim || k > kMaxDim)
        return QW_ERROR_UNSUPPORTED;
    if (misaligned(x) || misaligned(q) || misaligned(scales) || misaligned(y))
        return QW_ERROR_MISALIGNED;
    const uint64_t ybytes = (uint64_t)m * (uint64_t)n * 2u;
    if (overlaps(y, ybytes, x, (uint64_t)m * (uint64_t)k * 2u) ||
        overlaps(y, ybytes, q, (uint64_t)n * (uint64_t)k) ||
        overlaps(y, ybytes, scales, (uint64_t)n * 2u))
        return QW_ERROR_INVALID_VALUE;
    return QW_SUCCESS;
}

// Outlier slots per row that always suffice for the type-7 bound: the
// elements above it lie among the k - 1 - floor(pos) largest
// (pos = (pct / 100) (k - 1) in binary64); none at pct = 100.
int64_t outlier_capacity(int64_t k, double clip_percentile)
{
    if (clip_percentile == 100.0)
        return 0;
    const double frac_of_range = clip_percentile / 100.0;
    const double pos = frac_of_range * (double)(k - 1);
    const int64_t i = (int64_t)floor(pos);
    return i >= k - 1 ? 0 : k - 1 - i;
}

// Shared body of the fp32 and fp16 quantizer entry points (wbytes = bytes
// per input weight), with optional outlier side lists (fp32 only).
qw_status quantize_common(const void *w, int wbytes, int64_t n, int64_t k, double clip_percentile,
                          int8_t *q, uint16_t *scales, void *stream,
                          qw::OutlierSlots ol = qw::OutlierSlots{nullptr, nullptr, 0})
{
    if (n < 0 || k <= 0)
        return QW_ERROR_INVALID_VALUE;
    if (!(clip_percentile > 0.0 && clip_percentile <= 100.0)) // also rejects NaN
        return QW_ERROR_INVALID_VALUE;
    if (n == 0)
        return QW_SUCCESS;
    if (!w || !q || !scales)
        return QW_ERROR_INVALID_VALUE;
    if (k % 16 != 0 || k > QW_QUANTIZE_MAX_K || n > kMaxDim)
        return QW_ERROR_UNSUPPORTED;
    if (misaligned(w) || misaligned(q) || misaligned(scales))
        return QW_ERROR_MISALIGNED;
    const uint64_t elems = (uint64_t)n * (uint64_t)k;
    if (overlaps(q, elems, w, elems * (uint64_t)wbytes) ||
        overlaps(scales, (uint64_t)n * 2u, w, elems * (uint64_t)wbytes) ||
        overlaps(scales, (uint64_t)n * 2u, q, elems))
        return QW_ERROR_INVALID_VALUE;
    if (ol.idx != nullptr || ol.val != nullptr) {
        if (!ol.idx || !ol.val || ol.cap < 0 || wbytes != 4)
            return QW_ERROR_INVALID_VALUE;
        if (ol.cap < outlier_capacity(k, clip_percentile) || ol.cap > k)
            return QW_ERROR_INVALID_VALUE;
        if (misaligned(ol.idx) || misaligned(ol.val))
            return QW_ERROR_MISALIGNED;
        const uint64_t sb = (uint64_t)n * (uint64_t)ol.cap * 4u;
        const void *outs[3] = {q, scales, ol.val};
        const uint64_t outb[3] = {elems, (uint64_t)n * 2u, sb};
        if (overlaps(ol.idx, sb, w, elems * 4u) || overlaps(ol.val, sb, w, elems * 4u))
            return QW_ERROR_INVALID_VALUE;
        for (int i = 0; i < 3; ++i)
            if (overlaps(ol.idx, sb, outs[i], outb[i]) || (i < 2 && overlaps(ol.val, sb, outs[i], outb[i])))
                return QW_ERROR_INVALID_VALUE;
        if (ol.cap == 0)
            ol = qw::OutlierSlots{nullptr, nullptr, 0};
    }

    // Clip position of the type-7 percentile, in binary64 on the host:
    // pos = (pct / 100) * (k - 1), i = floor(pos), f = pos - i.
    int mode = 0;
    int64_t rank_i = k - 1;
    double frac_f = 0.0;
    if (clip_percentile != 100.0) {
        const double frac_of_range = clip_percentile / 100.0;
        const double pos = frac_of_range * (double)(k - 1); // no FMA: built with -ffp-contract=off
        const double i_floor = floor(pos);
        if ((int64_t)i_floor < k - 1) {
            mode = 1;
            rank_i = (int64_t)i_floor;
            frac_f = pos - i_floor;
        }
    }
    return launch_status(qw::launch_quantize(w, wbytes == 2, n, k, mode, rank_i, frac_f, nullptr, q,
                                             scales, nullptr, ol, static_cast<hipStream_t>(stream)));
}

// Shared body of the W8A16 entry points (zeros == nullptr: symmetric;
// ol.idx == nullptr: no outlier side lists).
qw_status gemm_common(const uint16_t *x, const int8_t *q, const uint16_t *scales, const int8_t *zeros,
                      uint16_t *y, int64_t m, int64_t n, int64_t k, int path, void *stream,
                      qw::OutlierList ol = qw::OutlierList{nullptr, nullptr, 0}, int tile = 0)
{
    if (path != QW_PATH_AUTO && path != QW_PATH_GEMV && path != QW_PATH_MFMA &&
        path != QW_PATH_SKINNY)
        return QW_ERROR_INVALID_VALUE;
    bool noop = false;
    const qw_status st = check_gemm_args(x, q, scales, y, m, n, k, noop);
    if (st != QW_SUCCESS || noop)
        return st;
    if (zeros) {
        if (misaligned(zeros))
            return QW_ERROR_MISALIGNED;
        if (overlaps(y, (uint64_t)m * (uint64_t)n * 2u, zeros, (uint64_t)n))
            return QW_ERROR_INVALID_VALUE;
    }
    if (ol.idx != nullptr) {
        const uint64_t sb = (uint64_t)n * (uint64_t)ol.cap * 4u;
        if (misaligned(ol.idx) || misaligned(ol.val))
            return QW_ERROR_MISALIGNED;
        if (overlaps(y, (uint64_t)m * (uint64_t)n * 2u, ol.idx, sb) ||
            overlaps(y, (uint64_t)m * (uint64_t)n * 2u, ol.val, sb))
            return QW_ERROR_INVALID_VALUE;
        if (ol.cap == 0)
            ol = qw::OutlierList{nullptr, nullptr, 0};
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (path == QW_PATH_AUTO) {
        // a tuning record for this shape bucket wins over the heuristic
        const int tuned = qw::tuned_choice(m, n, k);
        const int tpath = tuned / qw::kChoicePath;
        if (tuned >= 0 && (tpath != QW_PATH_GEMV || qw::gemv_supported(m, k)) &&
            (tpath != QW_PATH_MFMA || ((ol.idx == nullptr || ol.cap <= qw::kMfmaOutlierSlots) &&
                                       k <= qw::kMfmaMaxK &&
                                       (tuned % qw::kChoicePath != 256256 || k <= qw::kPingPongMaxK))) &&
            (tpath != QW_PATH_SKINNY || m <= 16 * 65535))
            return launch_status(qw::launch_choice(tuned, x, q, scales, zeros, ol, y, m, n, k, s));
        path = qw::auto_path(m, n, k);
        // side lists wider than the MFMA kernel stages in LDS: skinny kernel
        if (path == QW_PATH_MFMA && ol.idx != nullptr && ol.cap > qw::kMfmaOutlierSlots)
            path = QW_PATH_SKINNY;
    }
    if (path == QW_PATH_MFMA && ((ol.idx != nullptr && ol.cap > qw::kMfmaOutlierSlots) || k > qw::kMfmaMaxK))
        return QW_ERROR_UNSUPPORTED;
    if (path == QW_PATH_GEMV) {
        if (!qw::gemv_supported(m, k))
            return QW_ERROR_UNSUPPORTED;
        return launch_status(qw::launch_gemv(x, q, scales, zeros, ol, y, m, n, k, s));
    }
    if (path == QW_PATH_SKINNY) {
        if (m > 16 * 65535) // grid.y holds one 16-row activation tile per block row
            return QW_ERROR_UNSUPPORTED;
        return launch_status(qw::launch_skinny_gemm(x, q, scales, zeros, ol, y, m, n, k, s));
    }
    if (tile != 0)
        return launch_status(qw::launch_mfma_gemm_tile(tile, x, q, scales, zeros, ol, y, m, n, k, s));
    return launch_status(qw::launch_mfma_gemm(x, q, scales, zeros, ol, y, m, n, k, s));
}

} // namespace

extern "C" {

QW_API qw_status qw_quantize_weights(const float *w, int64_t n, int64_t k, double clip_percentile,
                                     int8_t *q, uint16_t *scales, void *stream)
{
    return quantize_common(w, 4, n, k, clip_percentile, q, scales, stream);
}

QW_API qw_status qw_quantize_weights_f16(const uint16_t *w, int64_t n, int64_t k, double clip_percentile,
                                         int8_t *q, uint16_t *scales, void *stream)
{
    return quantize_common(w, 2, n, k, clip_percentile, q, scales, stream);
}

QW_API int64_t qw_outlier_capacity(int64_t k, double clip_percentile)
{
    if (k <= 0 || !(clip_percentile > 0.0 && clip_percentile <= 100.0))
        return -1;
    return outlier_capacity(k, clip_percentile);
}

QW_API qw_status qw_quantize_weights_outliers(const float *w, int64_t n, int64_t k, double clip_percentile,
                                              int8_t *q, uint16_t *scales, int32_t *ol_idx, float *ol_val,
                                              int64_t cap, void *stream)
{
    if (n < 0 || k <= 0 || cap < 0)
        return QW_ERROR_INVALID_VALUE;
    if (n > 0 && (!ol_idx || !ol_val))
        return QW_ERROR_INVALID_VALUE;
    if (cap > k || cap > kMaxDim)
        return QW_ERROR_INVALID_VALUE;
    return quantize_common(w, 4, n, k, clip_percentile, q, scales, stream,
                           qw::OutlierSlots{ol_idx, ol_val, (int)cap});
}

QW_API qw_status qw_quantize_weights_fixed_range(const float *w, int64_t n, int64_t k,
                                                 const float *bounds, int8_t *q, uint16_t *scales,
                                                 void *stream)
{
    if (n < 0 || k <= 0)
        return QW_ERROR_INVALID_VALUE;
    if (n == 0)
        return QW_SUCCESS;
    if (!w || !bounds || !q || !scales)
        return QW_ERROR_INVALID_VALUE;
    if (k % 16 != 0 || k > QW_QUANTIZE_MAX_K || n > kMaxDim)
        return QW_ERROR_UNSUPPORTED;
    if (misaligned(w) || misaligned(bounds) || misaligned(q) || misaligned(scales))
        return QW_ERROR_MISALIGNED;
    const uint64_t elems = (uint64_t)n * (uint64_t)k;
    if (overlaps(q, elems, w, elems * 4u) || overlaps(scales, (uint64_t)n * 2u, w, elems * 4u) ||
        overlaps(scales, (uint64_t)n * 2u, q, elems) || overlaps(q, elems, bounds, (uint64_t)n * 4u) ||
        overlaps(scales, (uint64_t)n * 2u, bounds, (uint64_t)n * 4u))
        return QW_ERROR_INVALID_VALUE;
    return launch_status(qw::launch_quantize(w, false, n, k, 2, 0, 0.0, bounds, q, scales, nullptr,
                                             qw::OutlierSlots{nullptr, nullptr, 0}, static_cast<hipStream_t>(stream)));
}

QW_API qw_status qw_quantize_weights_asym(const float *w, int64_t n, int64_t k, int8_t *q,
                                          uint16_t *scales, int8_t *zeros, void *stream)
{
    if (n < 0 || k <= 0)
        return QW_ERROR_INVALID_VALUE;
    if (n == 0)
        return QW_SUCCESS;
    if (!w || !q || !scales || !zeros)
        return QW_ERROR_INVALID_VALUE;
    if (k % 16 != 0 || k > QW_QUANTIZE_MAX_K || n > kMaxDim)
        return QW_ERROR_UNSUPPORTED;
    if (misaligned(w) || misaligned(q) || misaligned(scales) || misaligned(zeros))
        return QW_ERROR_MISALIGNED;
    const uint64_t elems = (uint64_t)n * (uint64_t)k, nn = (uint64_t)n;
    if (overlaps(q, elems, w, elems * 4u) || overlaps(scales, nn * 2u, w, elems * 4u) ||
        overlaps(zeros, nn, w, elems * 4u) || overlaps(scales, nn * 2u, q, elems) ||
        overlaps(zeros, nn, q, elems) || overlaps(zeros, nn, scales, nn * 2u))
        return QW_ERROR_INVALID_VALUE;
    return launch_status(qw::launch_quantize(w, false, n, k, 3, 0, 0.0, nullptr, q, scales, zeros,
                                             qw::OutlierSlots{nullptr, nullptr, 0}, static_cast<hipStream_t>(stream)));
}

QW_API qw_status qw_w8a16_gemm_path(const uint16_t *x, const int8_t *q, const uint16_t *scales,
                                    uint16_t *y, int64_t m, int64_t n, int64_t k, int path,
                                    void *stream)
{
    return gemm_common(x, q, scales, nullptr, y, m, n, k, path, stream);
}

QW_API qw_status qw_w8a16_gemm_asym_path(const uint16_t *x, const int8_t *q, const uint16_t *scales,
                                         const int8_t *zeros, uint16_t *y, int64_t m, int64_t n,
                                         int64_t k, int path, void *stream)
{
    if (m > 0 && n > 0 && !zeros)
        return QW_ERROR_INVALID_VALUE;
    return gemm_common(x, q, scales, zeros, y, m, n, k, path, stream);
}

QW_API qw_status qw_w8a16_gemm_outliers_path(const uint16_t *x, const int8_t *q, const uint16_t *scales,
                                             const int32_t *ol_idx, const float *ol_val, int64_t cap,
                                             uint16_t *y, int64_t m, int64_t n, int64_t k, int path,
                                             void *stream)
{
    if (cap < 0 || cap > k || cap > kMaxDim)
        return QW_ERROR_INVALID_VALUE;
    if (m > 0 && n > 0 && cap > 0 && (!ol_idx || !ol_val))
        return QW_ERROR_INVALID_VALUE;
    return gemm_common(x, q, scales, nullptr, y, m, n, k, path, stream,
                       qw::OutlierList{cap > 0 ? ol_idx : nullptr, ol_val, (int)cap});
}

QW_API qw_status qw_w8a16_gemm_tile(const uint16_t *x, const int8_t *q, const uint16_t *scales,
                                    const int8_t *zeros, const int32_t *ol_idx, const float *ol_val,
                                    int64_t cap, uint16_t *y, int64_t m, int64_t n, int64_t k, int tile,
                                    void *stream)
{
    if (tile != 256256 && tile != 256128 && tile != 256064 && tile != 128128 && tile != 128064)
        return QW_ERROR_INVALID_VALUE;
    if (cap < 0 || cap > k || cap > kMaxDim || (zeros != nullptr && cap > 0))
        return QW_ERROR_INVALID_VALUE;
    if (m > 0 && n > 0 && cap > 0 && (!ol_idx || !ol_val))
        return QW_ERROR_INVALID_VALUE;
    if (tile == 256256 && k > qw::kPingPongMaxK && k % 16 == 0)
        return QW_ERROR_UNSUPPORTED;
    return gemm_common(x, q, scales, zeros, y, m, n, k, QW_PATH_MFMA, stream,
                       qw::OutlierList{cap > 0 ? ol_idx : nullptr, ol_val, (int)cap}, tile);
}

QW_API qw_status qw_w8a16_gemm_outliers(const uint16_t *x, const int8_t *q, const uint16_t *scales,
                                        const int32_t *ol_idx, const float *ol_val, int64_t cap,
                                        uint16_t *y, int64_t m, int64_t n, int64_t k, void *stream)
{
    return qw_w8a16_gemm_outliers_path(x, q, scales, ol_idx, ol_val, cap, y, m, n, k, QW_PATH_AUTO, stream);
}

QW_API qw_status qw_w8a16_gemm_asym(const uint16_t *x, const int8_t *q, const uint16_t *scales,
                                    const int8_t *zeros, uint16_t *y, int64_t m, int64_t n, int64_t k,
                                    void *stream)
{
    return qw_w8a16_gemm_asym_path(x, q, scales, zeros, y, m, n, k, QW_PATH_AUTO, stream);
}

QW_API qw_status qw_w8a16_gemm(const uint16_t *x, const int8_t *q, const uint16_t *scales,
                               uint16_t *y, int64_t m, int64_t n, int64_t k, void *stream)
{
    return qw_w8a16_gemm_path(x, q, scales, y, m, n, k, QW_PATH_AUTO, stream);
}

QW_API int qw_w8a16_gemm_auto_path(int64_t m, int64_t n, int64_t k)
{
    if (m < 0 || n < 0 || k <= 0 || k % 16 != 0)
        return -1;
    const int tuned = qw::tuned_choice(m, n, k);
    if (tuned >= 0 && (tuned / qw::kChoicePath != QW_PATH_GEMV || qw::gemv_supported(m, k)))
        return tuned / qw::kChoicePath;
    return qw::auto_path(m, n, k);
}

QW_API qw_status qw_w8a16_gemm_tune(const uint16_t *x, const int8_t *q, const uint16_t *scales, uint16_t *y,
                                    int64_t m, int64_t n, int64_t k, void *stream)
{
    bool noop = false;
    const qw_status st = check_gemm_args(x, q, scales, y, m, n, k, noop);
    if (st != QW_SUCCESS || noop)
        return st;
    int best = -1;
    const hipError_t e = qw::tune_gemm(x, q, scales, y, m, n, k, static_cast<hipStream_t>(stream), best);
    if (e != hipSuccess)
        return QW_ERROR_LAUNCH;
    qw::record_tuned_choice(m, n, k, best);
    return QW_SUCCESS;
}

QW_API int qw_w8a16_gemm_tuned_choice(int64_t m, int64_t n, int64_t k)
{
    if (m <= 0 || n <= 0 || k <= 0 || k % 16 != 0)
        return -1;
    return qw::tuned_choice(m, n, k);
}

QW_API void qw_w8a16_gemm_tune_reset(void)
{
    qw::reset_tuned_choices();
}

QW_API int qw_w8a16_gemm_mfma_tile(int64_t m, int64_t n, int64_t k)
{
    if (m <= 0 || n <= 0 || k <= 0 || k % 16 != 0 || m > kMaxDim || n > kMaxDim || k > kMaxDim)
        return -1;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return -1;
    const int tuned = qw::tuned_choice(m, n, k);
    if (tuned >= 0 && tuned / qw::kChoicePath == QW_PATH_MFMA)
        return tuned % qw::kChoicePath;
    return qw::mfma_tile_choice(m, n, k);
}

} // extern "C"

namespace {

// Argument checks shared by the W8A8 entry points; noop: nothing to do.
qw_status check_w8a8_args(const int8_t *qx, const uint16_t *sx, const int8_t *q, const uint16_t *scales,
                          const uint16_t *y, int64_t m, int64_t n, int64_t k, bool &noop)
{
    noop = false;
    if (m < 0 || n < 0 || k <= 0)
        return QW_ERROR_INVALID_VALUE;
    if (m == 0 || n == 0) {
        noop = true;
        return QW_SUCCESS;
    }
    if (!qx || !sx || !q || !scales || !y)
        return QW_ERROR_INVALID_VALUE;
    if (k % 16 != 0 || m > kMaxDim || n > kMaxDim || k > QW_W8A8_MAX_K)
        return QW_ERROR_UNSUPPORTED;
    if (misaligned(qx) || misaligned(sx) || misaligned(q) || misaligned(scales) || misaligned(y))
        return QW_ERROR_MISALIGNED;
    const uint64_t ybytes = (uint64_t)m * (uint64_t)n * 2u;
    if (overlaps(y, ybytes, qx, (uint64_t)m * (uint64_t)k) || overlaps(y, ybytes, sx, (uint64_t)m * 2u) ||
        overlaps(y, ybytes, q, (uint64_t)n * (uint64_t)k) || overlaps(y, ybytes, scales, (uint64_t)n * 2u))
        return QW_ERROR_INVALID_VALUE;
    return QW_SUCCESS;
}

} // namespace

extern "C" {

QW_API qw_status qw_w8a8_gemm_path(const int8_t *qx, const uint16_t *sx, const int8_t *q,
                                   const uint16_t *scales, uint16_t *y, int64_t m, int64_t n, int64_t k,
                                   int path, void *stream)
{
    if (path != QW_PATH_AUTO && path != QW_PATH_MFMA && path != QW_PATH_SKINNY)
        return QW_ERROR_INVALID_VALUE;
    bool noop = false;
    const qw_status st = check_w8a8_args(qx, sx, q, scales, y, m, n, k, noop);
    if (st != QW_SUCCESS || noop)
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (path == QW_PATH_AUTO) {
        // a tuning record for this shape bucket wins over the shape rule
        const int tuned = qw::tuned_choice(m, n, k, true);
        if (tuned >= 0 && (tuned / qw::kChoicePath != QW_PATH_SKINNY || m <= 16 * 65535))
            return launch_status(qw::launch_choice_w8a8(tuned, qx, sx, q, scales, y, m, n, k, s));
        path = qw::auto_path_w8a8(m, n, k);
    }
    if (path == QW_PATH_SKINNY) {
        if (m > 16 * 65535) // grid.y holds one 16-row activation tile per block row
            return QW_ERROR_UNSUPPORTED;
        return launch_status(qw::launch_w8a8_skinny(qx, sx, q, scales, y, m, n, k, s));
    }
    return launch_status(qw::launch_w8a8_gemm(qx, sx, q, scales, y, m, n, k, s));
}

QW_API qw_status qw_w8a8_gemm_tile(const int8_t *qx, const uint16_t *sx, const int8_t *q,
                                   const uint16_t *scales, uint16_t *y, int64_t m, int64_t n, int64_t k,
                                   int tile, void *stream)
{
    if (tile != 256256 && tile != 256128 && tile != 256064 && tile != 128064)
        return QW_ERROR_INVALID_VALUE;
    bool noop = false;
    const qw_status st = check_w8a8_args(qx, sx, q, scales, y, m, n, k, noop);
    if (st != QW_SUCCESS || noop)
        return st;
    return launch_status(
        qw::launch_w8a8_gemm_tile(tile, qx, sx, q, scales, y, m, n, k, static_cast<hipStream_t>(stream)));
}

QW_API qw_status qw_w8a8_gemm(const int8_t *qx, const uint16_t *sx, const int8_t *q,
                              const uint16_t *scales, uint16_t *y, int64_t m, int64_t n, int64_t k,
                              void *stream)
{
    return qw_w8a8_gemm_path(qx, sx, q, scales, y, m, n, k, QW_PATH_AUTO, stream);
}

QW_API int qw_w8a8_gemm_auto_path(int64_t m, int64_t n, int64_t k)
{
    if (m < 0 || n < 0 || k <= 0 || k % 16 != 0 || m > kMaxDim || n > kMaxDim || k > QW_W8A8_MAX_K)
        return -1;
    const int tuned = qw::tuned_choice(m, n, k, true);
    if (tuned >= 0)
        return tuned / qw::kChoicePath;
    return qw::auto_path_w8a8(m, n, k);
}

QW_API int qw_w8a8_gemm_mfma_tile(int64_t m, int64_t n, int64_t k)
{
    if (m <= 0 || n <= 0 || k <= 0 || k % 16 != 0 || m > kMaxDim || n > kMaxDim || k > QW_W8A8_MAX_K)
        return -1;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return -1;
    const int tuned = qw::tuned_choice(m, n, k, true);
    if (tuned >= 0 && tuned / qw::kChoicePath == QW_PATH_MFMA)
        return tuned % qw::kChoicePath;
    return qw::w8a8_tile_choice(m, n, k);
}

QW_API qw_status qw_w8a8_gemm_tune(const int8_t *qx, const uint16_t *sx, const int8_t *q, const uint16_t *scales,
                                   uint16_t *y, int64_t m, int64_t n, int64_t k, void *stream)
{
    bool noop = false;
    const qw_status st = check_w8a8_args(qx, sx, q, scales, y, m, n, k, noop);
    if (st != QW_SUCCESS || noop)
        return st;
    int best = -1;
    const hipError_t e = qw::tune_w8a8(qx, sx, q, scales, y, m, n, k, static_cast<hipStream_t>(stream), best);
    if (e != hipSuccess)
        return QW_ERROR_LAUNCH;
    qw::record_tuned_choice(m, n, k, best, true);
    return QW_SUCCESS;
}

QW_API int qw_w8a8_gemm_tuned_choice(int64_t m, int64_t n, int64_t k)
{
    if (m <= 0 || n <= 0 || k <= 0 || k % 16 != 0)
        return -1;
    return qw::tuned_choice(m, n, k, true);
}

QW_API qw_status qw_probe_stream_read(const void *p, int64_t bytes, uint32_t magic, uint32_t *sink, void *stream)
{
    if (bytes < 0)
        return QW_ERROR_INVALID_VALUE;
    if (bytes < 1024)
        return QW_SUCCESS;
    if (p == nullptr || sink == nullptr)
        return QW_ERROR_INVALID_VALUE;
    if (misaligned(p))
        return QW_ERROR_MISALIGNED;
    return launch_status(qw::launch_stream_read(p, bytes, magic, sink, static_cast<hipStream_t>(stream)));
}

QW_API qw_status qw_probe_shader_clock(uint64_t *out, void *stream)
{
    if (out == nullptr)
        return QW_ERROR_INVALID_VALUE;
    if ((reinterpret_cast<uintptr_t>(out) & 7u) != 0)
        return QW_ERROR_MISALIGNED;
    return launch_status(qw::launch_shader_clock(out, static_cast<hipStream_t>(stream)));
}

QW_API const char *qw_status_string(qw_status status)
{
    // C callers may pass any int; reading it through the enum type would be
    // undefined for values outside the enumeration, so read its bytes
    static_assert(sizeof(qw_status) == sizeof(int), "qw_status is int-sized");
    int code = 0;
    memcpy(&code, &status, sizeof code);
    switch (code) {
    case QW_SUCCESS:
        return "success";
    case QW_ERROR_INVALID_VALUE:
        return "invalid value (null pointer, negative size, k == 0, bad percentile or overlapping buffers)";
    case QW_ERROR_MISALIGNED:
        return "misaligned pointer (16-byte alignment required)";
    case QW_ERROR_UNSUPPORTED:
        return "unsupported size (k % 16 != 0 or a size beyond the documented maximum)";
    case QW_ERROR_LAUNCH:
        return "kernel launch failed";
    }
    return "unknown status";
}

QW_API int qw_version(void)
{
    return 100; // 0.1.0
}

} // extern "C"

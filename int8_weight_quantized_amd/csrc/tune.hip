// tune.hip -- per-shape kernel autotuning for the W8A16 and W8A8 GEMMs.
//
// The LightSeq article (section on quantized inference speed) reports int8
// GEMMs slower than fp16 at some shapes until each shape's GEMM was tuned
// automatically, and the LightSeq deck (TVM part) searches kernel
// parameters per dynamic shape with the token count padded to a multiple of
// 8.  Here the search space is the kernel (GEMV, skinny, MFMA) and the MFMA
// tile shape; a tuning call times every candidate on the caller's buffers
// and stream and records the fastest for the shape bucket (device, n, k,
// m rounded up to a multiple of 8; the W8A16 and W8A8 GEMMs keep separate
// records).  The automatic kernel choice of every entry point consults
// these records first.
//
// The records are the library's only mutable host state: a small map under
// a mutex, kept until the process ends or qw_w8a16_gemm_tune_reset.  No
// device memory is allocated; timing uses HIP events on the caller's
// stream, so a tuning call synchronizes with that stream.
#include <stdint.h>

#include <map>
#include <mutex>
#include <tuple>

#include "qw.h"
#include "qw_internal.h"

namespace qw {
namespace {

std::mutex g_tune_mutex;
// (dev, W8A8, n, k, m8) -> choice
std::map<std::tuple<int, bool, int64_t, int64_t, int64_t>, int> g_tuned;

int64_t bucket_m(int64_t m)
{
    return (m + 7) / 8 * 8;
}

} // namespace

int tuned_choice(int64_t m, int64_t n, int64_t k, bool a8)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return -1;
    std::lock_guard<std::mutex> lock(g_tune_mutex);
    const auto it = g_tuned.find(std::make_tuple(dev, a8, n, k, bucket_m(m)));
    return it == g_tuned.end() ? -1 : it->second;
}

void record_tuned_choice(int64_t m, int64_t n, int64_t k, int choice, bool a8)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return;
    std::lock_guard<std::mutex> lock(g_tune_mutex);
    g_tuned[std::make_tuple(dev, a8, n, k, bucket_m(m))] = choice;
}

void reset_tuned_choices()
{
    std::lock_guard<std::mutex> lock(g_tune_mutex);
    g_tuned.clear();
}

hipError_t launch_choice(int choice, const uint16_t *x, const int8_t *q, const uint16_t *scales,
                         const int8_t *zeros, OutlierList ol, uint16_t *y, int64_t m, int64_t n, int64_t k,
                         hipStream_t stream)
{
    const int path = choice / kChoicePath;
    const int tile = choice % kChoicePath;
    if (path == QW_PATH_GEMV)
        return launch_gemv(x, q, scales, zeros, ol, y, m, n, k, stream);
    if (path == QW_PATH_SKINNY)
        return launch_skinny_gemm(x, q, scales, zeros, ol, y, m, n, k, stream);
    return launch_mfma_gemm_tile(tile, x, q, scales, zeros, ol, y, m, n, k, stream);
}

hipError_t launch_choice_w8a8(int choice, const int8_t *qx, const uint16_t *sx, const int8_t *q,
                              const uint16_t *scales, uint16_t *y, int64_t m, int64_t n, int64_t k,
                              hipStream_t stream)
{
    if (choice / kChoicePath == QW_PATH_SKINNY)
        return launch_w8a8_skinny(qx, sx, q, scales, y, m, n, k, stream);
    return launch_w8a8_gemm_tile(choice % kChoicePath, qx, sx, q, scales, y, m, n, k, stream);
}

namespace {

// Times every candidate with launch(choice) on the caller's stream and sets
// best to the fastest; then runs the winner once more, leaving its result.
// Candidates are timed round-robin, one launch each per round, so that
// clock ramp-up and drift under load hit every candidate alike (timed one
// after another, the first candidates ran at a lower clock and the ranking
// followed the order); two untimed rounds first, then the median of seven.
template <class Launch>
hipError_t time_candidates(const int *cands, int nc, hipStream_t stream, Launch &&launch, int &best)
{
    hipEvent_t ev[2];
    if (hipEventCreate(&ev[0]) != hipSuccess)
        return hipErrorOutOfMemory;
    if (hipEventCreate(&ev[1]) != hipSuccess) {
        (void)hipEventDestroy(ev[0]);
        return hipErrorOutOfMemory;
    }
    constexpr int kWarm = 2, kRounds = 7;
    float times[8][kRounds];
    hipError_t err = hipSuccess;
    for (int r = 0; r < kWarm + kRounds && err == hipSuccess; ++r) {
        for (int c = 0; c < nc && err == hipSuccess; ++c) {
            const bool timed = r >= kWarm;
            if (timed)
                err = hipEventRecord(ev[0], stream);
            if (err == hipSuccess)
                err = launch(cands[c]);
            if (timed && err == hipSuccess)
                err = hipEventRecord(ev[1], stream);
            if (timed && err == hipSuccess)
                err = hipEventSynchronize(ev[1]);
            if (timed && err == hipSuccess)
                err = hipEventElapsedTime(&times[c][r - kWarm], ev[0], ev[1]);
        }
    }
    best = -1;
    float best_ms = 0.0f;
    for (int c = 0; c < nc && err == hipSuccess; ++c) {
        float *t = times[c];
        for (int a = 1; a < kRounds; ++a) // insertion sort; the median decides
            for (int b = a; b > 0 && t[b] < t[b - 1]; --b) {
                const float tmp = t[b];
                t[b] = t[b - 1];
                t[b - 1] = tmp;
            }
        const float ms = t[kRounds / 2];
        if (best < 0 || ms < best_ms) {
            best = cands[c];
            best_ms = ms;
        }
    }
    (void)hipEventDestroy(ev[0]);
    (void)hipEventDestroy(ev[1]);
    if (err != hipSuccess)
        return err;
    return launch(best);
}

} // namespace

hipError_t tune_gemm(const uint16_t *x, const int8_t *q, const uint16_t *scales, uint16_t *y, int64_t m,
                     int64_t n, int64_t k, hipStream_t stream, int &best)
{
    int cands[8];
    int nc = 0;
    if (gemv_supported(m, k))
        cands[nc++] = QW_PATH_GEMV * kChoicePath;
    if (m <= 16 * 65535)
        cands[nc++] = QW_PATH_SKINNY * kChoicePath;
    if (k <= kPingPongMaxK)
        cands[nc++] = QW_PATH_MFMA * kChoicePath + 256256;
    if (k <= kMfmaMaxK)
        for (int tile : {256128, 256064, 128128, 128064})
            cands[nc++] = QW_PATH_MFMA * kChoicePath + tile;
    const OutlierList none{nullptr, nullptr, 0};
    return time_candidates(cands, nc, stream, [&](int choice) {
        return launch_choice(choice, x, q, scales, nullptr, none, y, m, n, k, stream);
    }, best);
}

hipError_t tune_w8a8(const int8_t *qx, const uint16_t *sx, const int8_t *q, const uint16_t *scales, uint16_t *y,
                     int64_t m, int64_t n, int64_t k, hipStream_t stream, int &best)
{
    // the int8 kernels: the skinny kernel and the four W8A8 MFMA tiles (the
    // int8 128 x 128 tile is not built)
    int cands[5];
    int nc = 0;
    if (m <= 16 * 65535)
        cands[nc++] = QW_PATH_SKINNY * kChoicePath;
    for (int tile : {256256, 256128, 256064, 128064})
        cands[nc++] = QW_PATH_MFMA * kChoicePath + tile;
    return time_candidates(cands, nc, stream, [&](int choice) {
        return launch_choice_w8a8(choice, qx, sx, q, scales, y, m, n, k, stream);
    }, best);
}

} // namespace qw

// qw_internal.h -- host-side launchers shared between the translation units
// of libqw.  Arguments reaching these functions have been validated by the
// C ABI layer (qw_api.hip); the launchers only pick a kernel configuration
// and enqueue it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qw.h"

namespace qw {

// Per-row outlier side lists in ELL form: `cap` slots per row, columns in
// ascending order, unused slots column -1 and value 0 (idx == nullptr: no
// side lists).
struct OutlierSlots {
    int32_t *idx;
    float *val;
    int cap;
};
struct OutlierList {
    const int32_t *idx;
    const float *val;
    int cap;
};
// Side-list slots per row the MFMA kernel stages in LDS; wider lists go to
// the skinny kernel.
constexpr int kMfmaOutlierSlots = 4;
// Longest row the MFMA kernel takes: its per-lane copy offsets within a
// tile (at most 256 rows x k bytes) and a tile's byte range stay below 2^31.
// Longer rows go to the skinny kernel, which indexes in 64 bits.
constexpr int64_t kMfmaMaxK = QW_MFMA_MAX_K;

// Activation rows the skinny kernel covers per pass over the weights (32
// where it runs two 16-row activation tiles per wave, else 16).
int skinny_rows_per_pass(int64_t m, int64_t k);
static_assert(256 * kMfmaMaxK <= (int64_t(1) << 31) && 255 * kMfmaMaxK + 64 < (int64_t(1) << 31),
              "MFMA in-tile offsets");

// Per-row quantizer of fp32 (w_is_f16 false) or fp16 weights.  mode 0:
// absmax bound; mode 1: percentile bound with the rank i (0-based,
// ascending) and interpolation fraction f computed on the host in binary64
// (i < k - 1 in mode 1); mode 2 (fp32 weights only): the bound of row r is
// bounds[r] (device pointer, unused in the other modes); mode 3 (fp32
// weights only): asymmetric, range [min(0, min w), max(0, max w)], int8
// zero point per row written to zeros.  With ol.idx set (modes 0 and 1,
// fp32 weights): the elements above the bound go to the side lists and
// their codes are 0 (rows whose scale is 0 keep none).
hipError_t launch_quantize(const void *w, bool w_is_f16, int64_t n, int64_t k, int mode,
                           int64_t rank_i, double frac_f, const float *bounds, int8_t *q,
                           uint16_t *scales, int8_t *zeros, OutlierSlots ol, hipStream_t stream);

// The three W8A16 kernels take an optional per-row int8 zero point
// (`zeros`, nullptr for symmetric weights): the weight is then
// S[n] * (q[n][k] - z[n]); and optional outlier side lists (ol.idx ==
// nullptr: none), whose entries are added exactly: y += x[col] * value.

// Decode GEMV (VALU dot products).  Requires m <= 8 and
// m * ceil(k / 1024) <= 32 (the activations fit the LDS budget).
bool gemv_supported(int64_t m, int64_t k);
hipError_t launch_gemv(const uint16_t *x, const int8_t *q, const uint16_t *scales, const int8_t *zeros,
                       OutlierList ol, uint16_t *y, int64_t m, int64_t n, int64_t k, hipStream_t stream);

// Skinny MFMA GEMM: weights dequantized in registers, any m (intended for
// m <= 32), n, k with k % 16 == 0.
hipError_t launch_skinny_gemm(const uint16_t *x, const int8_t *q, const uint16_t *scales,
                              const int8_t *zeros, OutlierList ol, uint16_t *y, int64_t m, int64_t n,
                              int64_t k, hipStream_t stream);

// Kernel the automatic path picks for a shape (QW_PATH_* value).
int auto_path(int64_t m, int64_t n, int64_t k);

// MFMA tiled GEMM, any m, n, k with k % 16 == 0.
hipError_t launch_mfma_gemm(const uint16_t *x, const int8_t *q, const uint16_t *scales,
                            const int8_t *zeros, OutlierList ol, uint16_t *y, int64_t m, int64_t n,
                            int64_t k, hipStream_t stream);

// Output tile of the MFMA GEMM for this shape on the current device,
// encoded BN * 1000 + BM (256256: the 8-wave ping-pong kernel).
int mfma_tile_choice(int64_t m, int64_t n, int64_t k);

// Longest reduction of the 256 x 256 ping-pong tile: its 256-row activation
// tile spans 256 * k * 2 bytes of one buffer range, kept below 2^31.
constexpr int64_t kPingPongMaxK = QW_PINGPONG_MAX_K;
static_assert(256 * kPingPongMaxK * 2 <= (int64_t(1) << 31), "ping-pong buffer range");

// W8A8 GEMM on the matrix cores (int8 activation codes qx [m, k] with one
// fp16 scale per row in sx), any m, n, k with k % 16 == 0, and its tile.
hipError_t launch_w8a8_gemm(const int8_t *qx, const uint16_t *sx, const int8_t *q,
                            const uint16_t *scales, uint16_t *y, int64_t m, int64_t n, int64_t k,
                            hipStream_t stream);
int w8a8_tile_choice(int64_t m, int64_t n, int64_t k);
// W8A8 skinny kernel (int8 MFMA on the skinny kernel's layout) for a few
// activation rows, any m, n, k with k % 16 == 0.
hipError_t launch_w8a8_skinny(const int8_t *qx, const uint16_t *sx, const int8_t *q, const uint16_t *scales,
                              uint16_t *y, int64_t m, int64_t n, int64_t k, hipStream_t stream);

// Compute units of the current device (cached per device).
int device_cu_count();

// Measurement aids (probe.hip): a plain streaming read of `bytes` (a
// multiple of 1 KiB is read; the rest is ignored), and the shader clock
// measured over a short spin (out[0] shader-clock ticks, out[1] ticks of
// the 100 MHz constant clock).
hipError_t launch_stream_read(const void *p, int64_t bytes, uint32_t magic, uint32_t *sink, hipStream_t stream);
hipError_t launch_shader_clock(uint64_t *out, hipStream_t stream);

// Per-shape tuning records (tune.hip).  A choice encodes the kernel and the
// MFMA tile as path * kChoicePath + tile (tile 0 for GEMV and skinny).
constexpr int kChoicePath = 1000000;
// The W8A16 and W8A8 (a8) GEMMs keep separate records.
int tuned_choice(int64_t m, int64_t n, int64_t k, bool a8 = false); // -1: none
void record_tuned_choice(int64_t m, int64_t n, int64_t k, int choice, bool a8 = false);
void reset_tuned_choices();
hipError_t launch_choice(int choice, const uint16_t *x, const int8_t *q, const uint16_t *scales,
                         const int8_t *zeros, OutlierList ol, uint16_t *y, int64_t m, int64_t n, int64_t k,
                         hipStream_t stream);
// Times every candidate on the caller's buffers and stream (synchronizes
// with it) and returns the fastest in `best`; y holds the winner's result.
hipError_t tune_gemm(const uint16_t *x, const int8_t *q, const uint16_t *scales, uint16_t *y, int64_t m,
                     int64_t n, int64_t k, hipStream_t stream, int &best);
// The same for the W8A8 GEMM (skinny kernel and the int8 MFMA tiles).
hipError_t tune_w8a8(const int8_t *qx, const uint16_t *sx, const int8_t *q, const uint16_t *scales, uint16_t *y,
                     int64_t m, int64_t n, int64_t k, hipStream_t stream, int &best);
hipError_t launch_choice_w8a8(int choice, const int8_t *qx, const uint16_t *sx, const int8_t *q,
                              const uint16_t *scales, uint16_t *y, int64_t m, int64_t n, int64_t k,
                              hipStream_t stream);
// The W8A8 MFMA GEMM with a given tile (256128, 256064 or 128064).
hipError_t launch_w8a8_gemm_tile(int tile, const int8_t *qx, const uint16_t *sx, const int8_t *q,
                                 const uint16_t *scales, uint16_t *y, int64_t m, int64_t n, int64_t k,
                                 hipStream_t stream);
// The MFMA GEMM with a given tile (BN * 1000 + BM); hipErrorInvalidValue for
// a tile that is not built or a k the tile does not take.
hipError_t launch_mfma_gemm_tile(int tile, const uint16_t *x, const int8_t *q, const uint16_t *scales,
                                 const int8_t *zeros, OutlierList ol, uint16_t *y, int64_t m, int64_t n,
                                 int64_t k, hipStream_t stream);

} // namespace qw

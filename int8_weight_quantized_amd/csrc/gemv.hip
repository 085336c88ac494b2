// gemv.hip -- W8A16 decode GEMV / skinny GEMM on the VALU (gfx950).
//
// Decode multiplies one (or a few) activation rows with the whole weight
// matrix, so the time goes into loading the weights, and casting and scaling
// them can hide under that load ("探索ChatGLM2在算能BM1684X上INT8量化部署",
// section 4, the small-left-matrix argument and the prefill/decode
// discussion).  Here the int8 weights are streamed from HBM exactly once
// with 16-byte nontemporal loads, dequantized in registers with an exact
// byte-permute trick, and dotted with fp16 activations on v_dot2_f32_f16
// (fp32 accumulation).  The per-channel scale multiplies the fp32 sum.
//
// Work split.  The grid is sized to what the chip holds at once (W waves,
// at most WPC per CU, W chosen so that every wave gets the same number of
// RU-row groups); wave w owns rows w, w + W, w + 2W, ..., walked RU rows at
// a time, so at any moment the waves of the chip read one compact
// window of rows (DRAM page locality) instead of W scattered streams.  For
// one row, lane l reads bytes [c*1024 + 16 l, +16) for every 1 KiB chunk c:
// each load instruction of the wave covers 1 KiB of one row, fully
// coalesced.  An item is RU rows x CH chunks: its RU x CH 16-byte loads are
// all issued before any is consumed; the grid keeps 16 waves per CU so the
// chip holds plenty of bytes in flight.  X (m rows, fp16) is staged once
// per workgroup in LDS, after the first item's loads have been issued.  The RU*M per-lane partial sums are combined with a
// transposing butterfly (about RU*M shuffles instead of 6*RU*M).
//
// LDS layout of X: [m][chunk][half h][lane] x 16 bytes, where entry
// (m, c, h, l) holds x[m][c*1024 + 16 l + 8 h .. +7].  Lane l reads
// consecutive 16-byte slots for h = 0 and h = 1: no bank conflicts.
#include "qw_device.h"
#include "qw_internal.h"

#include <algorithm>

namespace qw {
namespace {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / kWave;
constexpr int kChunkK = kWave * 16; // k values covered by one wave-wide 16-byte load
constexpr int kGemvMaxMChunks = 32; // LDS budget: 32 * 2 KiB = 64 KiB
constexpr int64_t kLdsPerCu = 160 * 1024;

template <int MT, int RU, int CH>
struct GemvItem {
    u32x4_t w[RU][CH];
};

template <int MT, int RU, int CH>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(
    const uint16_t *__restrict__ x, const int8_t *__restrict__ q,
    const uint16_t *__restrict__ scales, const int8_t *__restrict__ zeros, OutlierList ol,
    uint16_t *__restrict__ y, int m, int n, int k, int chunks, int total_waves)
{
    extern __shared__ u32x4_t xs[];
    const int tid = threadIdx.x;
    const int lane = __lane_id();
    const int wave = tid / kWave;
    const int gw = blockIdx.x * kGemvWaves + wave;

    // this wave's rows gw + j * total_waves, j < my_rows; an item is RU of
    // them x CH chunks
    const int my_rows = gw < n ? (n - 1 - gw) / total_waves + 1 : 0;
    const int groups = (my_rows + RU - 1) / RU;
    const int batches = (chunks + CH - 1) / CH;
    const int items = gw < total_waves ? groups * batches : 0;

    auto issue = [&](int it, GemvItem<MT, RU, CH> &dst) {
        const int g = it / batches;
        const int b = it - g * batches;
#pragma unroll
        for (int r = 0; r < RU; ++r) {
#pragma unroll
            for (int cc = 0; cc < CH; ++cc) {
                const int c = b * CH + cc;
                const int kk = c * kChunkK + lane * 16;
                const int j = g * RU + r;
                const int64_t row = gw + (int64_t)j * total_waves;
                dst.w[r][cc] = (u32x4_t){0u, 0u, 0u, 0u};
                if (j < my_rows && kk < k)
                    dst.w[r][cc] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4_t *>(q + row * k + kk));
            }
        }
    };

    GemvItem<MT, RU, CH> buf;
    if (items > 0)
        issue(0, buf);

    // ---- stage X into LDS (rows m..MT-1 are zero) while the loads fly ----
    const int entries = MT * chunks * 2 * kWave;
    for (int e = tid; e < entries; e += kGemvThreads) {
        const int l = e % kWave;
        const int h = (e / kWave) & 1;
        const int mc = e / (2 * kWave);
        const int c = mc % chunks;
        const int mm = mc / chunks;
        const int kk = c * kChunkK + l * 16 + h * 8;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (mm < m && kk < k)
            v = *reinterpret_cast<const u32x4_t *>(x + (int64_t)mm * k + kk);
        xs[e] = v;
    }
    __syncthreads();

    constexpr int R = RU * MT;
    float acc[R];
    half2_t zbias[RU];

    auto consume = [&](int it, const GemvItem<MT, RU, CH> &cur) {
        const int g = it / batches;
        const int b = it - g * batches;
        if (b == 0) {
#pragma unroll
            for (int i = 0; i < R; ++i)
                acc[i] = 0.0f;
            // asymmetric weights: the zero points of this item's rows
#pragma unroll
            for (int r = 0; r < RU; ++r) {
                const int j = g * RU + r;
                const int64_t row = gw + (int64_t)j * total_waves;
                zbias[r] = zero_point_bias(zeros != nullptr && j < my_rows ? (int)zeros[row] : 0);
            }
        }
#pragma unroll
        for (int cc = 0; cc < CH; ++cc) {
            const int c = b * CH + cc;
            if (c < chunks) {
                half2_t xv[MT][8];
#pragma unroll
                for (int mm = 0; mm < MT; ++mm) {
                    const u32x4_t a = xs[((mm * chunks + c) * 2 + 0) * kWave + lane];
                    const u32x4_t bb = xs[((mm * chunks + c) * 2 + 1) * kWave + lane];
                    xv[mm][0] = as_half2(a.x);
                    xv[mm][1] = as_half2(a.y);
                    xv[mm][2] = as_half2(a.z);
                    xv[mm][3] = as_half2(a.w);
                    xv[mm][4] = as_half2(bb.x);
                    xv[mm][5] = as_half2(bb.y);
                    xv[mm][6] = as_half2(bb.z);
                    xv[mm][7] = as_half2(bb.w);
                }
#pragma unroll
                for (int r = 0; r < RU; ++r) {
                    half2_t hw[8];
                    i8x16_to_half2x8(cur.w[r][cc], hw, zbias[r]);
#pragma unroll
                    for (int mm = 0; mm < MT; ++mm) {
                        float a = acc[r * MT + mm];
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            a = dot2(hw[j], xv[mm][j], a);
                        acc[r * MT + mm] = a;
                    }
                }
            }
        }
        if (b == batches - 1) {
            butterfly_reduce<R>(acc);
            if ((lane & (kWave / R - 1)) == 0) {
                const int idx = butterfly_index<R>(lane);
                const int r = idx / MT;
                const int mm = idx % MT;
                const int j = g * RU + r;
                const int64_t row = gw + (int64_t)j * total_waves;
                if (j < my_rows && mm < m) {
                    const float s = f16_bits_to_f32(scales[row]);
                    float out = acc[0] * s;
                    // exact outliers of this row, with X from the LDS copy
                    // (entry e holds x[mm][c kChunkK + 16 l + 8 h + 0..7])
                    if (ol.idx != nullptr) {
                        const _Float16 *xh = reinterpret_cast<const _Float16 *>(xs);
                        for (int e = 0; e < ol.cap; ++e) {
                            const int kk = ol.idx[row * ol.cap + e];
                            if (kk < 0 || kk >= k)
                                break; // used slots come first
                            const int c = kk / kChunkK, l = (kk % kChunkK) / 16, h = (kk % 16) / 8;
                            const float xv = (float)xh[((((mm * chunks + c) * 2 + h) * kWave + l) * 8) + kk % 8];
                            out += xv * ol.val[row * ol.cap + e];
                        }
                    }
                    y[(int64_t)mm * n + row] = f32_to_f16_bits(out);
                }
            }
        }
    };

    // one item in flight per wave; the chip-wide occupancy (many resident
    // waves) keeps HBM busy, which measured faster than a two-deep per-wave
    // pipeline with fewer waves
    for (int it = 0; it < items; ++it) {
        if (it > 0)
            issue(it, buf);
        consume(it, buf);
    }
}

template <int MT, int RU, int CH, int WPC>
hipError_t launch_cfg(const uint16_t *x, const int8_t *q, const uint16_t *scales, const int8_t *zeros,
                      OutlierList ol, uint16_t *y,
                      int64_t m, int64_t n, int64_t k, hipStream_t stream)
{
    const int chunks = (int)((k + kChunkK - 1) / kChunkK);
    const size_t lds = (size_t)MT * chunks * 2 * kWave * sizeof(u32x4_t);
    // one wave per RU rows at most; otherwise about as many waves as the chip
    // keeps resident (WPC per CU), trimmed so that every wave walks the same
    // number of RU-row groups (no half-empty last round)
    const int64_t groups = (n + RU - 1) / RU;
    int64_t waves = groups;
    int64_t wpc = WPC;
    const int64_t lds_wgs = kLdsPerCu / (int64_t)lds; // workgroups one CU's LDS holds
    if (wpc > lds_wgs * kGemvWaves)
        wpc = lds_wgs * kGemvWaves;
    const int64_t cap = (int64_t)device_cu_count() * wpc;
    if (waves > cap) {
        const int64_t per = (groups + cap - 1) / cap;
        waves = (groups + per - 1) / per;
    }
    const int blocks = (int)((waves + kGemvWaves - 1) / kGemvWaves);
    hipLaunchKernelGGL((gemv_kernel<MT, RU, CH>), dim3(blocks), dim3(kGemvThreads), lds, stream,
                       x, q, scales, zeros, ol, y, (int)m, (int)n, (int)k, chunks, (int)waves);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Register-resident decode GEMV (m <= 2, k <= kStreamMaxChunks KiB).
//
// Each lane keeps its share of X in registers for the whole kernel: lane l
// takes k = c * 1024 + 16 l + [0, 16) of every 1 KiB chunk c, the same 16
// values that its 16-byte weight loads cover, so no LDS is touched in the
// main loop.  The grid is 8 waves per CU (trimmed so that every wave walks
// the same number of rows); wave w takes rows w, w + W, w + 2 W, ..., so
// that at any moment the chip streams one compact window of rows, and keeps
// two rows in flight: row t + 1's loads are issued before row t is
// consumed.  That is 8 KiB in flight per wave, 64 KiB per CU, the depth
// at which a plain streaming read of the same bytes peaks on MI355X.
//
// The cast's bias is folded per 16-code chunk: with h the fp16 value
// 1152 + q that the byte permute produces, and z the row's zero point
// (0 for symmetric weights),
//     sum_j x_j (q_j - z) = sum_j x_j h_j - (sum_j x_j 1152 + z sum_j x_j),
// where the sums run over the 16 codes of one load, each formed from zero
// by the same chain of v_dot2_f32_f16; the two sums of x alone are formed
// once per kernel from the registers of X.  That saves the two packed
// subtractions per four codes; the chunk difference is then added to the
// running sum.  The degenerate cases stay exact: a row of zero codes with
// z = 0 gives two bitwise equal chains and adds +0, z = 0 adds exactly
// nothing to the correction (so asymmetric weights with zero points of 0
// give the symmetric result bit for bit), and with integer inputs whose
// partial sums stay below 2^24 every step is exact.  The per-chunk chains
// sum 16 terms of at most 1279 |x|, so their rounding stays far below the
// fp16 rounding of Y.
// ---------------------------------------------------------------------------

constexpr int kStreamMaxChunks = 8; // k <= 8192: X takes 8 VGPRs per chunk and row
constexpr int kStreamWavesPerCu = 8;

template <int MT, int CH, bool ZP>
__global__ __launch_bounds__(256) void gemv_stream_kernel(
    const uint16_t *__restrict__ x, const int8_t *__restrict__ q, const uint16_t *__restrict__ scales,
    const int8_t *__restrict__ zeros, OutlierList ol, uint16_t *__restrict__ y, int m, int n, int k, int waves)
{
    const int lane = __lane_id();
    const int gw = blockIdx.x * kGemvWaves + threadIdx.x / kWave;
    if (gw >= waves)
        return;
    // this lane's X: xr[mm][c][j] = x[mm][c * 1024 + 16 lane + 2 j + {0, 1}]
    half2_t xr[MT][CH][8];
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int kk = c * kChunkK + lane * 16;
            u32x4_t a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
            if (mm < m && kk < k) {
                a = *reinterpret_cast<const u32x4_t *>(x + (int64_t)mm * k + kk);
                b = *reinterpret_cast<const u32x4_t *>(x + (int64_t)mm * k + kk + 8);
            }
            xr[mm][c][0] = as_half2(a.x); xr[mm][c][1] = as_half2(a.y);
            xr[mm][c][2] = as_half2(a.z); xr[mm][c][3] = as_half2(a.w);
            xr[mm][c][4] = as_half2(b.x); xr[mm][c][5] = as_half2(b.y);
            xr[mm][c][6] = as_half2(b.z); xr[mm][c][7] = as_half2(b.w);
        }
    }
    // the bias chains sum_j x_j 1152 of each chunk, and (ZP) the sums of x
    float corr[MT][CH], sx[MT][CH];
    {
        const half2_t b = (half2_t){(_Float16)1152.0f, (_Float16)1152.0f};
        const half2_t one = (half2_t){(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int mm = 0; mm < MT; ++mm)
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                float a = 0.0f, e = 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    a = dot2(b, xr[mm][c][j], a);
                    if constexpr (ZP)
                        e = dot2(one, xr[mm][c][j], e);
                }
                corr[mm][c] = a;
                sx[mm][c] = e;
            }
    }
    constexpr int R = MT; // partial sums per row: one per activation row
    const int rows = (n - 1 - gw) / waves + 1;
    const int mine = butterfly_index<R>(lane); // the activation row this lane writes (R > 1)
    // a row in flight: its codes, and its scale and zero point (loaded with
    // the codes, so that the epilogue does not wait for another load)
    struct Row {
        u32x4_t w[CH];
        uint16_t s;
        int8_t z;
    };
    // Lanes past the end of a ragged last chunk load the row's last 16
    // codes instead (a valid address, no branch around the load); their X is
    // zero, so those codes add exactly zero to both chains.
    int koff[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c)
        koff[c] = min(c * kChunkK + lane * 16, k - 16);
    auto issue = [&](int t, Row &b) {
        const int8_t *qr = q + (gw + (int64_t)t * waves) * k;
        const int64_t row = gw + (int64_t)t * waves;
#pragma unroll
        for (int c = 0; c < CH; ++c)
            b.w[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(qr + koff[c]));
        b.s = scales[row];
        b.z = ZP ? zeros[row] : (int8_t)0;
    };
    auto consume = [&](int t, const Row &b) {
        const int64_t row = gw + (int64_t)t * waves;
        float acc[R];
#pragma unroll
        for (int mm = 0; mm < MT; ++mm)
            acc[mm] = 0.0f;
        const float zf = (float)b.z;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            // the byte permute of i8x4_to_half2x2 without its subtraction:
            // hw holds 1152 + q exactly
            half2_t hw[8];
            const uint32_t wv[4] = {b.w[c].x, b.w[c].y, b.w[c].z, b.w[c].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t u = wv[e] ^ 0x80808080u;
                hw[2 * e] = as_half2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u));
                hw[2 * e + 1] = as_half2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u));
            }
#pragma unroll
            for (int mm = 0; mm < MT; ++mm) {
                float a = 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    a = dot2(hw[j], xr[mm][c][j], a);
                const float cb = ZP ? corr[mm][c] + zf * sx[mm][c] : corr[mm][c];
                acc[mm] += a - cb;
            }
        }
        butterfly_reduce<R>(acc);
        if ((lane & (kWave / R - 1)) == 0 && mine < m) {
            float out = acc[0] * f16_bits_to_f32(b.s);
            // exact outliers of this row, with X read from global memory
            if (ol.idx != nullptr) {
                for (int e = 0; e < ol.cap; ++e) {
                    const int kk = ol.idx[row * ol.cap + e];
                    if (kk < 0 || kk >= k)
                        break; // used slots come first
                    out += f16_bits_to_f32(x[(int64_t)mine * k + kk]) * ol.val[row * ol.cap + e];
                }
            }
            y[(int64_t)mine * n + row] = f32_to_f16_bits(out);
        }
    };
    // two rows in flight: row t + 1's loads go out before row t is consumed.
    // The steady loop is unrolled by two (each buffer a fixed register set)
    // and issues unconditionally, so that the compiler can count the loads in
    // flight and waits only for the row it consumes; the last one or two
    // rows are handled after it.
    // (A scheduling barrier after each issue keeps the compiler from sinking
    // the next row's loads below the start of the current row's arithmetic.)
    Row b0, b1;
    issue(0, b0);
    int t = 0;
    for (; t + 2 < rows; t += 2) {
        issue(t + 1, b1);
        __builtin_amdgcn_sched_barrier(0);
        consume(t, b0);
        issue(t + 2, b0);
        __builtin_amdgcn_sched_barrier(0);
        consume(t + 1, b1);
    }
    if (t + 1 < rows) {
        issue(t + 1, b1);
        consume(t, b0);
        consume(t + 1, b1);
    } else {
        consume(t, b0);
    }
}

template <int MT, int CH>
hipError_t launch_stream(const uint16_t *x, const int8_t *q, const uint16_t *scales, const int8_t *zeros,
                         OutlierList ol, uint16_t *y, int64_t m, int64_t n, int64_t k, hipStream_t stream)
{
    // about 8 waves per CU, trimmed so that every wave walks the same number of rows
    int64_t waves = std::min<int64_t>(n, (int64_t)device_cu_count() * kStreamWavesPerCu);
    const int64_t per = (n + waves - 1) / waves;
    waves = (n + per - 1) / per;
    const int blocks = (int)((waves + kGemvWaves - 1) / kGemvWaves);
    if (zeros == nullptr)
        hipLaunchKernelGGL((gemv_stream_kernel<MT, CH, false>), dim3(blocks), dim3(kGemvThreads), 0, stream, x, q,
                           scales, zeros, ol, y, (int)m, (int)n, (int)k, (int)waves);
    else
        hipLaunchKernelGGL((gemv_stream_kernel<MT, CH, true>), dim3(blocks), dim3(kGemvThreads), 0, stream, x, q,
                           scales, zeros, ol, y, (int)m, (int)n, (int)k, (int)waves);
    return hipGetLastError();
}

template <int MT>
hipError_t launch_stream_chunks(const uint16_t *x, const int8_t *q, const uint16_t *scales, const int8_t *zeros,
                                OutlierList ol, uint16_t *y, int64_t m, int64_t n, int64_t k, hipStream_t stream)
{
    switch ((k + kChunkK - 1) / kChunkK) {
    case 1: return launch_stream<MT, 1>(x, q, scales, zeros, ol, y, m, n, k, stream);
    case 2: return launch_stream<MT, 2>(x, q, scales, zeros, ol, y, m, n, k, stream);
    case 3: return launch_stream<MT, 3>(x, q, scales, zeros, ol, y, m, n, k, stream);
    case 4: return launch_stream<MT, 4>(x, q, scales, zeros, ol, y, m, n, k, stream);
    case 5: return launch_stream<MT, 5>(x, q, scales, zeros, ol, y, m, n, k, stream);
    case 6: return launch_stream<MT, 6>(x, q, scales, zeros, ol, y, m, n, k, stream);
    case 7: return launch_stream<MT, 7>(x, q, scales, zeros, ol, y, m, n, k, stream);
    default: return launch_stream<MT, 8>(x, q, scales, zeros, ol, y, m, n, k, stream);
    }
}

} // namespace

bool gemv_supported(int64_t m, int64_t k)
{
    if (m < 1 || m > 8)
        return false;
    const int64_t chunks = (k + kChunkK - 1) / kChunkK;
    int64_t mt = 1;
    while (mt < m)
        mt <<= 1;
    return mt * chunks <= kGemvMaxMChunks;
}

hipError_t launch_gemv(const uint16_t *x, const int8_t *q, const uint16_t *scales, const int8_t *zeros,
                       OutlierList ol, uint16_t *y,
                       int64_t m, int64_t n, int64_t k, hipStream_t stream)
{
    // decode: one or two activation rows held in registers.  (Four rows
    // measured 1.4-4x slower than the skinny kernel: the dot products per
    // weight byte grow with the rows and the VALU, not the stream, sets the
    // time.)
    if (m <= 2 && (k + kChunkK - 1) / kChunkK <= kStreamMaxChunks)
        return m <= 1 ? launch_stream_chunks<1>(x, q, scales, zeros, ol, y, m, n, k, stream)
                      : launch_stream_chunks<2>(x, q, scales, zeros, ol, y, m, n, k, stream);
    // otherwise X is staged in LDS; (MT, RU, CH, waves per CU) from measured
    // sweeps; WPC stays within what each configuration's register use lets a
    // CU hold at once
    if (m <= 1)
        return launch_cfg<1, 2, 4, 28>(x, q, scales, zeros, ol, y, m, n, k, stream);
    if (m <= 2)
        return launch_cfg<2, 1, 4, 32>(x, q, scales, zeros, ol, y, m, n, k, stream);
    if (m <= 4)
        return launch_cfg<4, 2, 2, 16>(x, q, scales, zeros, ol, y, m, n, k, stream);
    return launch_cfg<8, 2, 2, 16>(x, q, scales, zeros, ol, y, m, n, k, stream);
}

} // namespace qw

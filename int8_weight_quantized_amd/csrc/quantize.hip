// quantize.hip -- per-output-channel symmetric int8 weight quantizer (gfx950).
//
// Method: symmetric 8-bit quantization of each weight row onto codes
// [-127, 127] with an absmax bound or a percentage-clipped bound (LightSeq
// slide deck "LightSeq：高性能NLP序列推理实践", slides "量化流程" and
// "量化：裁剪+对称"), one F16 scale per output channel of a Linear weight
// ("探索ChatGLM2在算能BM1684X上INT8量化部署", sections 2 and 3).
//
// Input weights are fp32, or fp16 widened exactly to binary32 on load (the
// same arithmetic then follows).  One workgroup (one wave for rows up to
// 1024 values) owns one row.  The
// row is read from HBM exactly once with 16-byte loads and stays in
// registers (VPT float4 per thread) while the bound is found, so the kernel
// moves 4 bytes in and 1 byte out per weight plus 2 bytes of scale per row
// -- the HBM roofline of the operation.
//
//   absmax bound:      wave max-reductions of the |w| bit patterns (for
//                      non-negative binary32 values the integer order is
//                      the numeric order), then across waves through LDS.
//   percentile bound:  a[i] and a[i+1] of the sorted |w|.  Near the top
//                      (k - 1 - i <= 12, e.g. 99.9 and 99.99 for k <= 8192)
//                      by walking down the distinct values from the maximum,
//                      one block reduction per value; otherwise by an exact
//                      radix select of rank i over the |w| bit patterns, 4
//                      passes of 8 bits with a 256-bin LDS histogram, and
//                      a[i+1] from a count of values <= a[i] and a
//                      min-reduction of the values above it.  Interpolation
//                      in binary64 without FMA.
//
// Rounding contract: the scale is binary16(binary32(t / 127)) with true
// IEEE division; codes are clamp(rint(binary32(w / S)), -127, 127) where
// rint rounds half to even (v_rndne_f32).  This file is compiled with
// -ffp-contract=off and the pragma below so no multiply-add is fused.
#pragma clang fp contract(off)

#include "qw_device.h"
#include "qw_internal.h"

namespace qw {
namespace {

// descending ranks up to which the top-down walk replaces the radix select
constexpr uint32_t kTopDownMaxRank = 12;

template <int THREADS>
struct QuantShared {
    uint32_t red[THREADS / kWave];
    uint32_t red2[THREADS / kWave];
    uint32_t hist[256];
    uint32_t scan[256];
    uint32_t digit;
    uint32_t remaining;
};

template <int THREADS>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, QuantShared<THREADS> &sh)
{
    constexpr int W = THREADS / kWave;
    v = wave_max_u32(v);
    const int wave = threadIdx.x / kWave;
    if (__lane_id() == 0)
        sh.red[wave] = v;
    __syncthreads();
    uint32_t r = sh.red[0];
#pragma unroll
    for (int i = 1; i < W; ++i)
        r = sh.red[i] > r ? sh.red[i] : r;
    __syncthreads();
    return r;
}

// Sum of `a` and min of `b` over the block in one LDS round trip.
template <int THREADS>
__device__ __forceinline__ void block_sum_min_u32(uint32_t a, uint32_t b, QuantShared<THREADS> &sh,
                                                  uint32_t &sum, uint32_t &mn)
{
    constexpr int W = THREADS / kWave;
    a = wave_sum_u32(a);
    b = wave_min_u32(b);
    const int wave = threadIdx.x / kWave;
    if (__lane_id() == 0) {
        sh.red[wave] = a;
        sh.red2[wave] = b;
    }
    __syncthreads();
    sum = 0;
    mn = 0xffffffffu;
#pragma unroll
    for (int i = 0; i < W; ++i) {
        sum += sh.red[i];
        mn = sh.red2[i] < mn ? sh.red2[i] : mn;
    }
    __syncthreads();
}

// Inclusive prefix sum across the 64 lanes of a wave (log-step shuffles).
__device__ __forceinline__ uint32_t wave_inclusive_scan_u32(uint32_t v)
{
    const int lane = __lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t t = (uint32_t)__builtin_amdgcn_ds_bpermute(((lane - off) & (kWave - 1)) << 2, (int)v);
        v += lane >= off ? t : 0u;
    }
    return v;
}

// Clip percentiles near 100 need the elements of descending rank r and
// r - 1 (r = k - 1 - i small).  Walking down the distinct values from the
// maximum takes one block reduction per distinct value passed, far fewer
// barriers than a radix select: a level is the largest value below the
// previous one, and the count of its copies tells which descending ranks it
// covers.
__device__ __forceinline__ uint32_t abs_bits(float v);
template <int THREADS, int VPT>
__device__ void block_top_pair(const float (&v)[VPT * 4], const bool (&valid)[VPT], uint32_t r,
                               QuantShared<THREADS> &sh, uint32_t &ai, uint32_t &ai1)
{
    uint32_t mx = 0;
#pragma unroll
    for (int j = 0; j < VPT; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t x = valid[j] ? abs_bits(v[j * 4 + e]) : 0u;
            mx = x > mx ? x : mx;
        }
    uint32_t level = block_max_u32<THREADS>(mx, sh);
    uint32_t above = 0;       // elements strictly greater than `level`
    uint32_t prev = level;    // the level before (the next larger value)
    ai = ai1 = level;
    // every pass covers at least one more descending rank, so at most r + 1
    // passes run; the bound also caps the loop
    for (uint32_t pass = 0; pass <= r; ++pass) {
        uint32_t cnt = 0, below = 0;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            if (!valid[j])
                continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t x = abs_bits(v[j * 4 + e]);
                cnt += x == level ? 1u : 0u;
                below = (x < level && x > below) ? x : below;
            }
        }
        uint32_t total, inv_next;
        block_sum_min_u32<THREADS>(cnt, ~below, sh, total, inv_next);
        if (above + total > r) {
            // descending ranks above .. above + total - 1 hold `level`
            ai = level;
            ai1 = r - 1 >= above ? level : prev;
            return;
        }
        above += total;
        prev = level;
        level = ~inv_next;
    }
}

// Bit pattern of the element of 0-based ascending rank `rank` among the
// valid |w| patterns held by the block (radix select, 8 bits per pass).
__device__ __forceinline__ uint32_t abs_bits(float v)
{
    return __builtin_bit_cast(uint32_t, v) & 0x7fffffffu; // |w| as ordered bits
}

template <int THREADS, int VPT>
__device__ uint32_t block_select_rank(const float (&v)[VPT * 4], const bool (&valid)[VPT],
                                      uint32_t rank, QuantShared<THREADS> &sh)
{
    // the first kBinThreads threads own BPT consecutive bins each
    constexpr int kBinThreads = THREADS < 256 ? THREADS : 256;
    constexpr int BPT = 256 / kBinThreads;
    static_assert(THREADS % kWave == 0 && 256 % kBinThreads == 0, "bin ownership");
    uint32_t prefix = 0, mask = 0, remaining = rank;
    const int tid = threadIdx.x;
#pragma unroll
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int b = tid; b < 256; b += THREADS)
            sh.hist[b] = 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            if (!valid[j])
                continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t x = abs_bits(v[j * 4 + e]);
                if ((x & mask) == prefix)
                    atomicAdd(&sh.hist[(x >> shift) & 255u], 1u);
            }
        }
        __syncthreads();
        // inclusive scan of the 256 bins: each bin-owning wave scans its
        // threads' bin totals in registers, then adds the totals of the
        // waves before it
        uint32_t c[BPT], tot = 0, incl = 0;
        if (tid < kBinThreads) {
#pragma unroll
            for (int b = 0; b < BPT; ++b) {
                c[b] = sh.hist[tid * BPT + b];
                tot += c[b];
            }
            incl = wave_inclusive_scan_u32(tot);
            if (__lane_id() == kWave - 1)
                sh.scan[tid / kWave] = incl;
        }
        __syncthreads();
        if (tid < kBinThreads) {
            for (int w = 0; w < tid / kWave; ++w)
                incl += sh.scan[w];
            uint32_t excl = incl - tot;
#pragma unroll
            for (int b = 0; b < BPT; ++b) {
                if (excl <= remaining && remaining < excl + c[b]) {
                    sh.digit = (uint32_t)(tid * BPT + b);
                    sh.remaining = remaining - excl;
                }
                excl += c[b];
            }
        }
        __syncthreads();
        prefix |= sh.digit << shift;
        mask |= 255u << shift;
        remaining = sh.remaining;
        __syncthreads();
    }
    return prefix;
}

// Four consecutive weights of a row as binary32: 16 bytes of fp32, or 8
// bytes of fp16 widened exactly.
template <bool F16>
__device__ __forceinline__ float4_t load4(const void *row, int idx)
{
    if constexpr (F16) {
        const u32x2_t b = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(row) + idx);
        return (float4_t){f16_bits_to_f32((uint16_t)(b.x & 0xffffu)), f16_bits_to_f32((uint16_t)(b.x >> 16)),
                          f16_bits_to_f32((uint16_t)(b.y & 0xffffu)), f16_bits_to_f32((uint16_t)(b.y >> 16))};
    } else {
        return __builtin_nontemporal_load(reinterpret_cast<const float4_t *>(row) + idx);
    }
}

// MODE: 0 absmax bound, 1 percentile bound, 2 fixed range (the bound of
// row r is bounds[r], given by the caller; no reduction), 3 asymmetric
// (range [min(0, min w), max(0, max w)] over 255 steps, int8 zero point
// per row written to zeros).  OUTL: the elements above the bound are
// written to the row's outlier slots (ascending column) and get code 0.
template <int THREADS, int VPT, int MODE, bool F16, bool OUTL = false>
__global__ __launch_bounds__(THREADS) void quantize_rows_kernel(
    const void *__restrict__ w, int k, int64_t rank_i, double frac_f,
    const float *__restrict__ bounds, int8_t *__restrict__ q, uint16_t *__restrict__ scales,
    int8_t *__restrict__ zeros, OutlierSlots ol)
{
    constexpr bool PERCENTILE = MODE == 1;
    __shared__ QuantShared<THREADS> sh;
    const int64_t row = blockIdx.x;
    const int nvec = k >> 2;
    const void *src = static_cast<const uint8_t *>(w) + row * (int64_t)k * (F16 ? 2 : 4);

    float v[VPT * 4];
    bool valid[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int idx = threadIdx.x + j * THREADS;
        valid[j] = idx < nvec;
        float4_t f = {0.f, 0.f, 0.f, 0.f};
        if (valid[j])
            f = load4<F16>(src, idx);
        v[j * 4 + 0] = f.x;
        v[j * 4 + 1] = f.y;
        v[j * 4 + 2] = f.z;
        v[j * 4 + 3] = f.w;
    }
    float t;
    float neg_lo = 0.0f; // MODE 3: -min(0, min w)
    if constexpr (MODE == 2) {
        t = bounds[row];
    } else if constexpr (MODE == 3) {
        // max(0, max w) and max(0, max -w) as bit patterns of non-negative
        // floats, whose unsigned order is their numeric order
        uint32_t hb = 0, lb = 0;
#pragma unroll
        for (int e = 0; e < VPT * 4; ++e) {
            const float val = v[e];
            const uint32_t b = abs_bits(val);
            if (val > 0.0f)
                hb = b > hb ? b : hb;
            if (val < 0.0f)
                lb = b > lb ? b : lb;
        }
        t = __builtin_bit_cast(float, block_max_u32<THREADS>(hb, sh));
        neg_lo = __builtin_bit_cast(float, block_max_u32<THREADS>(lb, sh));
    } else if constexpr (!PERCENTILE) {
        uint32_t m = 0;
#pragma unroll
        for (int e = 0; e < VPT * 4; ++e) {
            const uint32_t x = abs_bits(v[e]);
            m = x > m ? x : m;
        }
        t = __builtin_bit_cast(float, block_max_u32<THREADS>(m, sh));
    } else {
        // rank_i < k - 1 here (the host sends i >= k - 1 down the absmax path)
        const uint32_t r = (uint32_t)((int64_t)k - 1 - rank_i);
        uint32_t ai, ai1;
        if (r <= kTopDownMaxRank) {
            block_top_pair<THREADS, VPT>(v, valid, r, sh, ai, ai1);
        } else {
            ai = block_select_rank<THREADS, VPT>(v, valid, (uint32_t)rank_i, sh);
            uint32_t le = 0, gt_min = 0xffffffffu;
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                if (!valid[j])
                    continue;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t x = abs_bits(v[j * 4 + e]);
                    le += x <= ai ? 1u : 0u;
                    if (x > ai && x < gt_min)
                        gt_min = x;
                }
            }
            uint32_t count_le, next_up;
            block_sum_min_u32<THREADS>(le, gt_min, sh, count_le, next_up);
            // a[i+1] equals a[i] when more than i+1 values are <= a[i]
            ai1 = ((uint64_t)rank_i + 1 < (uint64_t)count_le) ? ai : next_up;
        }
        const double lo = (double)__builtin_bit_cast(float, ai);
        const double hi = (double)__builtin_bit_cast(float, ai1);
        const double gap = __dsub_rn(hi, lo);
        const double step = __dmul_rn(frac_f, gap);
        t = (float)__dadd_rn(lo, step);
    }

    // symmetric: S = t / 127; asymmetric: S = (hi - lo) / 255, the range
    // over the 2^8 - 1 steps, and z shifts code -lo/S down to -128
    const float s32 = MODE == 3 ? __fdiv_rn(__fadd_rn(t, neg_lo), 255.0f) : __fdiv_rn(t, 127.0f);
    const uint16_t s16 = f32_to_f16_bits(s32);
    const float s = f16_bits_to_f32(s16);
    float zf = 0.0f;
    if constexpr (MODE == 3) {
        if (s != 0.0f) {
            zf = __builtin_rintf(__fdiv_rn(neg_lo, s)) - 128.0f;
            zf = zf > 127.0f ? 127.0f : zf;
            zf = zf < -128.0f ? -128.0f : zf;
        }
    }
    constexpr float kLo = MODE == 3 ? -128.0f : -127.0f;
    if (threadIdx.x == 0) {
        scales[row] = s16;
        if constexpr (MODE == 3)
            zeros[row] = (int8_t)(int)zf;
    }

    // Codes.  The contract is rint(binary32(w / s)); a true division per
    // weight costs about ten VALU instructions, so the quotient is first
    // estimated as w * rs with rs = binary32(1 / s).  That estimate is within
    // |w / s| * 2^-23 of the exact quotient (two roundings of 2^-24 each), so
    // for |w / s| < 256 within 2^-15.  rint of the estimate and rint of the
    // correctly rounded quotient can only differ when a half-integer lies
    // between them or the quotient rounds onto one; both require the
    // estimate to be within 2^-15 + ulp/2 of a half-integer.  Estimates
    // closer than 2^-12 to a half-integer therefore take the true division
    // (about one weight in four thousand).  |estimate| >= 256 clamps to
    // +-127 either way, as does an infinite one.
    const float rs = s != 0.0f ? __fdiv_rn(1.0f, s) : 0.0f;
    constexpr float kNearHalf = 1.0f / 4096.0f;
    uint32_t *dst = reinterpret_cast<uint32_t *>(q + row * (int64_t)k);
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int idx = threadIdx.x + j * THREADS;
        if (!valid[j])
            continue;
        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            int code = 0;
            const bool outlier = OUTL && __builtin_fabsf(v[j * 4 + e]) > t;
            if (s != 0.0f && !outlier) {
                const float est = v[j * 4 + e] * rs;
                float r = __builtin_rintf(est);
                // distance of est to the nearest half-integer (exact: est - r
                // is exact for |est| < 2^23, and so is the subtraction of 0.5)
                const float d = __builtin_fabsf(__builtin_fabsf(est - r) - 0.5f);
                if (__builtin_expect(d < kNearHalf && __builtin_fabsf(est) < 256.0f, 0))
                    r = __builtin_rintf(__fdiv_rn(v[j * 4 + e], s));
                r += zf; // exact: integers of magnitude below 2^24
                r = r > 127.0f ? 127.0f : r;
                r = r < kLo ? kLo : r;
                code = (int)r;
            }
            packed |= ((uint32_t)code & 0xffu) << (8 * e);
        }
        __builtin_nontemporal_store(packed, dst + idx);
    }

    if constexpr (OUTL) {
        // Compact the outliers into the row's slots in column order: slice
        // j of every thread covers columns 4 (tid + j THREADS) + [0, 4), so
        // slices in order and threads in order within a slice are columns in
        // order.  One block-wide exclusive scan of the per-thread counts per
        // slice; at most the host-checked capacity is ever reached (the
        // elements above the type-7 bound are among the k - 1 - i largest),
        // and the slot check below only guards the writes.
        int32_t *oi = ol.idx + row * (int64_t)ol.cap;
        float *ov = ol.val + row * (int64_t)ol.cap;
        const int wave = threadIdx.x / kWave;
        constexpr int W = THREADS / kWave;
        uint32_t base = 0;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            uint32_t mine = 0;
            if (s != 0.0f && valid[j]) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    mine += __builtin_fabsf(v[j * 4 + e]) > t ? 1u : 0u;
            }
            const uint32_t incl = wave_inclusive_scan_u32(mine);
            if (__lane_id() == kWave - 1)
                sh.red[wave] = incl;
            __syncthreads();
            uint32_t before = 0, total = 0;
#pragma unroll
            for (int wv = 0; wv < W; ++wv) {
                const uint32_t c = sh.red[wv];
                before += wv < wave ? c : 0u;
                total += c;
            }
            __syncthreads();
            uint32_t slot = base + before + incl - mine;
            if (mine != 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (__builtin_fabsf(v[j * 4 + e]) > t) {
                        if (slot < (uint32_t)ol.cap) {
                            oi[slot] = 4 * (threadIdx.x + j * THREADS) + e;
                            ov[slot] = v[j * 4 + e];
                        }
                        ++slot;
                    }
                }
            }
            base += total;
        }
        for (uint32_t p = base + threadIdx.x; p < (uint32_t)ol.cap; p += THREADS) {
            oi[p] = -1;
            ov[p] = 0.0f;
        }
    }
}

template <int THREADS, int VPT, bool F16>
hipError_t launch_typed(const void *w, int64_t n, int64_t k, int mode, int64_t rank_i, double frac_f,
                        const float *bounds, int8_t *q, uint16_t *scales, int8_t *zeros,
                        OutlierSlots ol, hipStream_t stream)
{
    const dim3 grid((unsigned)n), block(THREADS);
    if (ol.idx != nullptr) {
        if constexpr (F16) {
            return hipErrorInvalidValue; // side lists: fp32 weights only
        } else {
            if (mode == 0)
                hipLaunchKernelGGL((quantize_rows_kernel<THREADS, VPT, 0, false, true>), grid, block, 0, stream,
                                   w, (int)k, rank_i, frac_f, bounds, q, scales, zeros, ol);
            else if (mode == 1)
                hipLaunchKernelGGL((quantize_rows_kernel<THREADS, VPT, 1, false, true>), grid, block, 0, stream,
                                   w, (int)k, rank_i, frac_f, bounds, q, scales, zeros, ol);
            else
                return hipErrorInvalidValue;
            return hipGetLastError();
        }
    }
    if (mode == 0)
        hipLaunchKernelGGL((quantize_rows_kernel<THREADS, VPT, 0, F16>), grid, block, 0, stream,
                           w, (int)k, rank_i, frac_f, bounds, q, scales, zeros, ol);
    else if (mode == 1)
        hipLaunchKernelGGL((quantize_rows_kernel<THREADS, VPT, 1, F16>), grid, block, 0, stream,
                           w, (int)k, rank_i, frac_f, bounds, q, scales, zeros, ol);
    else if constexpr (F16)
        return hipErrorInvalidValue; // fixed range and asymmetric: fp32 weights only
    else if (mode == 2)
        hipLaunchKernelGGL((quantize_rows_kernel<THREADS, VPT, 2, false>), grid, block, 0, stream,
                           w, (int)k, rank_i, frac_f, bounds, q, scales, zeros, ol);
    else
        hipLaunchKernelGGL((quantize_rows_kernel<THREADS, VPT, 3, false>), grid, block, 0, stream,
                           w, (int)k, rank_i, frac_f, bounds, q, scales, zeros, ol);
    return hipGetLastError();
}

template <int THREADS, int VPT>
hipError_t launch_cfg(const void *w, bool f16, int64_t n, int64_t k, int mode, int64_t rank_i,
                      double frac_f, const float *bounds, int8_t *q, uint16_t *scales, int8_t *zeros,
                      OutlierSlots ol, hipStream_t stream)
{
    return f16 ? launch_typed<THREADS, VPT, true>(w, n, k, mode, rank_i, frac_f, bounds, q, scales, zeros, ol,
                                                  stream)
               : launch_typed<THREADS, VPT, false>(w, n, k, mode, rank_i, frac_f, bounds, q, scales, zeros, ol,
                                                   stream);
}

} // namespace

hipError_t launch_quantize(const void *w, bool w_is_f16, int64_t n, int64_t k, int mode,
                           int64_t rank_i, double frac_f, const float *bounds, int8_t *q,
                           uint16_t *scales, int8_t *zeros, OutlierSlots ol, hipStream_t stream)
{
    // float4 slots per row; a workgroup of THREADS holds THREADS * VPT of them.
    // Rows up to 1024 values get one wave each: every reduction is then a
    // wave reduction (measured 22% faster at 4096 x 1024, 99.99th
    // percentile; no gain at 2048).
    const int64_t nvec = k / 4;
    if (nvec <= kWave * 1)
        return launch_cfg<64, 1>(w, w_is_f16, n, k, mode, rank_i, frac_f, bounds, q, scales, zeros, ol, stream);
    if (nvec <= kWave * 2)
        return launch_cfg<64, 2>(w, w_is_f16, n, k, mode, rank_i, frac_f, bounds, q, scales, zeros, ol, stream);
    if (nvec <= kWave * 4)
        return launch_cfg<64, 4>(w, w_is_f16, n, k, mode, rank_i, frac_f, bounds, q, scales, zeros, ol, stream);
    if (nvec <= 256 * 1)
        return launch_cfg<256, 1>(w, w_is_f16, n, k, mode, rank_i, frac_f, bounds, q, scales, zeros, ol, stream);
    if (nvec <= 256 * 2)
        return launch_cfg<256, 2>(w, w_is_f16, n, k, mode, rank_i, frac_f, bounds, q, scales, zeros, ol, stream);
    if (nvec <= 256 * 4)
        return launch_cfg<256, 4>(w, w_is_f16, n, k, mode, rank_i, frac_f, bounds, q, scales, zeros, ol, stream);
    if (nvec <= 256 * 8)
        return launch_cfg<256, 8>(w, w_is_f16, n, k, mode, rank_i, frac_f, bounds, q, scales, zeros, ol, stream);
    if (nvec <= 256 * 16)
        return launch_cfg<256, 16>(w, w_is_f16, n, k, mode, rank_i, frac_f, bounds, q, scales, zeros, ol, stream);
    if (nvec <= 1024 * 8)
        return launch_cfg<1024, 8>(w, w_is_f16, n, k, mode, rank_i, frac_f, bounds, q, scales, zeros, ol, stream);
    return launch_cfg<1024, 16>(w, w_is_f16, n, k, mode, rank_i, frac_f, bounds, q, scales, zeros, ol, stream);
}

} // namespace qw

// gemm_mfma.hip -- W8A16 prefill GEMM on the matrix cores (gfx950).
//
// Prefill multiplies max_length activation rows with every weight, so the
// matmul itself dominates ("探索ChatGLM2在算能BM1684X上INT8量化部署",
// section 4: the W8A16 gain shrinks as max_length grows).  The int8 weight
// tile is read once per workgroup, cast to fp16 exactly in registers and
// written into LDS next to the fp16 activation tile; v_mfma_f32_16x16x32_f16
// contracts the two with fp32 accumulation; the per-channel scale
// multiplies the fp32 accumulators in the epilogue, which then rounds to
// fp16 and stores.
//
// Roles: the MFMA "A" operand is the weight tile (rows = output channels
// n), "B" is the activation tile (columns = activation rows m), so each
// lane ends up holding 4 consecutive output channels of one activation row
// and the epilogue stores 8 contiguous bytes of Y per lane.
//
// Tiling: BN x BM output tile per workgroup, BK = 64 per k step, 2x2 waves
// each owning a (BN/2) x (BM/2) sub-tile; the k loop is double-buffered in
// LDS with one barrier per step (the next tile's global loads are issued
// before the current tile's MFMAs and parked in registers).  Rows are
// padded by 16 bytes in LDS so the 16 lanes that read one 16-byte column
// slice hit distinct banks.  Workgroups are renumbered so that each XCD
// (dispatch is round-robin over the 8 XCDs) walks a contiguous run of
// tiles that share weight rows in its own L2.
#include "qw_device.h"
#include "qw_internal.h"

namespace qw {
namespace {

typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kGemmThreads = 256; // 2 x 2 waves

template <int BN, int BM, int BK>
struct TileCfg {
    static constexpr int kWavesN = 2, kWavesM = 2;
    static constexpr int kThreads = kWavesN * kWavesM * kWave;
    static_assert(kThreads == kGemmThreads, "launch bounds mismatch");
    static constexpr int kWaveN = BN / kWavesN; // output channels per wave
    static constexpr int kWaveM = BM / kWavesM; // activation rows per wave
    static constexpr int kSubN = kWaveN / 16;
    static constexpr int kSubM = kWaveM / 16;
    static constexpr int kLdsRow = BK + 8;      // halves per LDS row (16-byte pad)
    static constexpr int kWChunks = BN * BK / 16; // 16-byte int8 chunks of the W tile
    static constexpr int kXChunks = BM * BK / 8;  // 16-byte fp16 chunks of the X tile
    static constexpr int kWPerThread = kWChunks / kThreads;
    static constexpr int kXPerThread = kXChunks / kThreads;
    static_assert(kWChunks % kThreads == 0 && kXChunks % kThreads == 0, "tile/thread mismatch");
    static_assert(BK % 32 == 0, "BK must be a multiple of the MFMA k (32)");
};

__device__ __forceinline__ int xcd_remap(int bid, int nblocks)
{
    const int per = nblocks / 8, rem = nblocks % 8;
    const int xcd = bid % 8, local = bid / 8;
    return xcd * per + (xcd < rem ? xcd : rem) + local;
}

template <int BN, int BM, int BK>
__global__ __launch_bounds__(kGemmThreads) void mfma_gemm_kernel(
    const uint16_t *__restrict__ x, const int8_t *__restrict__ q,
    const uint16_t *__restrict__ scales, uint16_t *__restrict__ y,
    int m, int n, int k, int tiles_m, int tiles_n)
{
    using C = TileCfg<BN, BM, BK>;
    __shared__ _Float16 ws[2][BN][C::kLdsRow];
    __shared__ _Float16 xs[2][BM][C::kLdsRow];

    const int tid = threadIdx.x;
    const int lane = __lane_id();
    const int wave = tid / kWave;
    const int wave_n = wave % C::kWavesN;
    const int wave_m = wave / C::kWavesN;

    const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    const int tn = tile / tiles_m;
    const int tm = tile % tiles_m;
    const int n0 = tn * BN;
    const int m0 = tm * BM;

    const int ktiles = (k + BK - 1) / BK;

    u32x4_t wreg[C::kWPerThread];
    u32x4_t xreg[C::kXPerThread];

    auto load_tile = [&](int kt) {
        const int k0 = kt * BK;
#pragma unroll
        for (int i = 0; i < C::kWPerThread; ++i) {
            const int c = tid + i * C::kThreads;
            const int row = c / (BK / 16);
            const int kc = c % (BK / 16);
            const int gn = n0 + row;
            const int gk = k0 + kc * 16;
            wreg[i] = (u32x4_t){0u, 0u, 0u, 0u};
            if (gn < n && gk < k)
                wreg[i] = *reinterpret_cast<const u32x4_t *>(q + (int64_t)gn * k + gk);
        }
#pragma unroll
        for (int i = 0; i < C::kXPerThread; ++i) {
            const int c = tid + i * C::kThreads;
            const int row = c / (BK / 8);
            const int kc = c % (BK / 8);
            const int gm = m0 + row;
            const int gk = k0 + kc * 8;
            xreg[i] = (u32x4_t){0u, 0u, 0u, 0u};
            if (gm < m && gk < k)
                xreg[i] = *reinterpret_cast<const u32x4_t *>(x + (int64_t)gm * k + gk);
        }
    };

    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < C::kWPerThread; ++i) {
            const int c = tid + i * C::kThreads;
            const int row = c / (BK / 16);
            const int kc = c % (BK / 16);
            half2_t h[8];
            i8x16_to_half2x8(wreg[i], h);
            u32x4_t lo = {__builtin_bit_cast(uint32_t, h[0]), __builtin_bit_cast(uint32_t, h[1]),
                          __builtin_bit_cast(uint32_t, h[2]), __builtin_bit_cast(uint32_t, h[3])};
            u32x4_t hi = {__builtin_bit_cast(uint32_t, h[4]), __builtin_bit_cast(uint32_t, h[5]),
                          __builtin_bit_cast(uint32_t, h[6]), __builtin_bit_cast(uint32_t, h[7])};
            *reinterpret_cast<u32x4_t *>(&ws[buf][row][kc * 16]) = lo;
            *reinterpret_cast<u32x4_t *>(&ws[buf][row][kc * 16 + 8]) = hi;
        }
#pragma unroll
        for (int i = 0; i < C::kXPerThread; ++i) {
            const int c = tid + i * C::kThreads;
            const int row = c / (BK / 8);
            const int kc = c % (BK / 8);
            *reinterpret_cast<u32x4_t *>(&xs[buf][row][kc * 8]) = xreg[i];
        }
    };

    float4v acc[C::kSubN][C::kSubM];
#pragma unroll
    for (int i = 0; i < C::kSubN; ++i)
#pragma unroll
        for (int j = 0; j < C::kSubM; ++j)
            acc[i][j] = (float4v){0.f, 0.f, 0.f, 0.f};

    load_tile(0);
    store_tile(0);
    __syncthreads();

    const int lrow = lane % 16;
    const int lgrp = lane / 16;
    for (int kt = 0; kt < ktiles; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < ktiles)
            load_tile(kt + 1);
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            const int koff = ks * 32 + lgrp * 8;
            half8_t a[C::kSubN], b[C::kSubM];
#pragma unroll
            for (int i = 0; i < C::kSubN; ++i)
                a[i] = *reinterpret_cast<const half8_t *>(&ws[buf][wave_n * C::kWaveN + i * 16 + lrow][koff]);
#pragma unroll
            for (int j = 0; j < C::kSubM; ++j)
                b[j] = *reinterpret_cast<const half8_t *>(&xs[buf][wave_m * C::kWaveM + j * 16 + lrow][koff]);
#pragma unroll
            for (int i = 0; i < C::kSubN; ++i)
#pragma unroll
                for (int j = 0; j < C::kSubM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < ktiles)
            store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: scale, round to fp16, store ----
    const bool vec_ok = (n % 4) == 0;
#pragma unroll
    for (int i = 0; i < C::kSubN; ++i) {
        const int gn = n0 + wave_n * C::kWaveN + i * 16 + lgrp * 4;
        float s[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            s[r] = (gn + r < n) ? f16_bits_to_f32(scales[gn + r]) : 0.0f;
#pragma unroll
        for (int j = 0; j < C::kSubM; ++j) {
            const int gm = m0 + wave_m * C::kWaveM + j * 16 + lrow;
            if (gm >= m)
                continue;
            uint16_t out[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                out[r] = f32_to_f16_bits(acc[i][j][r] * s[r]);
            uint16_t *dst = y + (int64_t)gm * n + gn;
            if (vec_ok && gn + 3 < n) {
                u32x2_t pk = {(uint32_t)out[0] | ((uint32_t)out[1] << 16),
                              (uint32_t)out[2] | ((uint32_t)out[3] << 16)};
                *reinterpret_cast<u32x2_t *>(dst) = pk;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (gn + r < n)
                        dst[r] = out[r];
            }
        }
    }
}

template <int BN, int BM, int BK>
hipError_t launch_cfg(const uint16_t *x, const int8_t *q, const uint16_t *scales, uint16_t *y,
                      int64_t m, int64_t n, int64_t k, hipStream_t stream)
{
    using C = TileCfg<BN, BM, BK>;
    const int tiles_m = (int)((m + BM - 1) / BM);
    const int tiles_n = (int)((n + BN - 1) / BN);
    const int64_t blocks = (int64_t)tiles_m * tiles_n;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((mfma_gemm_kernel<BN, BM, BK>), dim3((unsigned)blocks), dim3(C::kThreads), 0,
                       stream, x, q, scales, y, (int)m, (int)n, (int)k, tiles_m, tiles_n);
    return hipGetLastError();
}

} // namespace

hipError_t launch_mfma_gemm(const uint16_t *x, const int8_t *q, const uint16_t *scales, uint16_t *y,
                            int64_t m, int64_t n, int64_t k, hipStream_t stream)
{
    if (m <= 32)
        return launch_cfg<128, 32, 64>(x, q, scales, y, m, n, k, stream);
    if (m <= 64)
        return launch_cfg<128, 64, 64>(x, q, scales, y, m, n, k, stream);
    return launch_cfg<128, 128, 64>(x, q, scales, y, m, n, k, stream);
}

} // namespace qw

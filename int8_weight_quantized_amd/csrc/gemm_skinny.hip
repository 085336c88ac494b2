// gemm_skinny.hip -- W8A16 skinny GEMM (a few activation rows) on the matrix
// cores (gfx950).
//
// Between decode (one token) and prefill (max_length tokens) the matmul has
// a handful of activation rows: the weight stream from HBM still sets the
// time ("探索ChatGLM2在算能BM1684X上INT8量化部署", section 4: small left
// matrix => bound by loading the right matrix), but the per-row VALU dot
// products of the GEMV path grow with m.  Here the contraction runs on
// v_mfma_f32_16x16x32_f16 instead: the int8 weights are cast to fp16 exactly
// in registers and used as the MFMA "A" operand; the activations are the "B"
// operand (16 columns, rows beyond m are zero).
//
// Work split: a workgroup of KSPLIT waves owns RT x 16 weight rows x MT x 16
// activation rows; wave w walks the k steps [w*S/KSPLIT, (w+1)*S/KSPLIT)
// of the S = ceil(k/64) steps of 64, four steps (256 codes of each row) per
// iteration.  The MFMA layout wants lane l (row r = l % 16, group
// g = l / 16) to hold bytes [64 s + 16 g, +16) of row r, which as a load
// would touch sixteen 64-byte row segments per instruction; instead each
// load instruction reads four rows x 256 contiguous bytes (16-byte
// nontemporal loads), the wave writes them into its own slice of LDS and
// reads them back in the MFMA layout (measured 12-25% faster).  Of the 16
// codes a lane holds per step, the first 8 feed one MFMA (k slots
// 8 g .. 8 g + 7 of a 32-wide k block), the last 8 a second one; the
// activation operand is loaded once with the same k assignment and reused
// by all RT row tiles, and each cast weight operand feeds the MFMAs of all
// MT activation tiles (so up to 16 MT activation rows take one pass over the
// weights).  KSPLIT is chosen so the grid has enough waves to
// keep HBM busy.  The KSPLIT partial tiles are summed in LDS in wave order
// (deterministic), then scaled (the scales are loaded at the start, so their
// latency hides under the main loop), rounded to fp16 and transposed
// through LDS, so that Y is written in whole 16-byte pieces of its rows.
#include "qw_device.h"
#include "qw_internal.h"

#include <type_traits>

namespace qw {
namespace {

typedef float float4v __attribute__((ext_vector_type(4)));
typedef int int4v __attribute__((ext_vector_type(4)));

constexpr int kSkinnyUnroll = 4;
constexpr int kSkinnyTargetWaves = 2048; // enough in-flight loads to fill HBM

// A8 (W8A8): the activations are int8 codes with one fp16 scale per row
// (sx); the 16 codes a lane holds per step are exactly the A operand of one
// v_mfma_i32_16x16x64_i8 (k slots 16 g .. 16 g + 15 of the 64-wide step),
// the activation codes the B operand with the same assignment, the
// accumulators are exact int32, and the epilogue scales by S[n] * Sx[m].
// Zero points and side lists are W8A16 only (null with A8).
template <int RT, int MT, int KSPLIT, bool A8 = false, bool ZP = false>
__global__ __launch_bounds__(KSPLIT * 64) void skinny_gemm_kernel(
    const void *__restrict__ xv, const uint16_t *__restrict__ sx, const int8_t *__restrict__ q,
    const uint16_t *__restrict__ scales, const int8_t *__restrict__ zeros, OutlierList ol,
    uint16_t *__restrict__ y, int m, int n, int k)
{
    const uint16_t *__restrict__ x = static_cast<const uint16_t *>(xv);
    using acc_t = std::conditional_t<A8, int4v, float4v>;
    // Per wave, a staging slice for the weight codes of one iteration:
    // [tile][row][256 bytes + 16 pad].  After the main loop the same memory
    // holds the partial tiles of waves 1 .. KSPLIT-1.
    constexpr int kStageRow = 64 * kSkinnyUnroll + 16; // 256 codes + pad
    constexpr int kStageBytes = KSPLIT * RT * 16 * kStageRow;
    constexpr int kPartialBytes = (KSPLIT > 1 ? KSPLIT - 1 : 1) * RT * MT * kWave * (int)sizeof(acc_t);
    __shared__ __attribute__((aligned(16))) uint8_t smem[kStageBytes > kPartialBytes ? kStageBytes : kPartialBytes];
    // the finished fp16 tile, [activation row][channel], padded rows
    __shared__ __attribute__((aligned(16))) uint16_t ytile[16 * MT][16 * RT + 8];
    static_assert(kSkinnyUnroll == 4, "one iteration covers 256 codes of a row");

    const int lane = __lane_id();
    const int wave = threadIdx.x / kWave;
    const int r = lane % 16;
    const int g = lane / 16;
    const int n0 = blockIdx.x * 16 * RT;
    const int m0 = blockIdx.y * 16 * MT;

    const int steps_total = (k + 63) / 64;
    const int s_begin = (int)(((int64_t)wave * steps_total) / KSPLIT);
    const int s_end = (int)(((int64_t)(wave + 1) * steps_total) / KSPLIT);

    const int8_t *qrow[RT];
    bool row_ok[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int row = n0 + 16 * t + r;
        row_ok[t] = row < n;
        qrow[t] = q + (int64_t)(row_ok[t] ? row : 0) * k;
    }
    // activation row m0 + 16 mt + r is what this lane feeds into the B
    // operand of activation tile mt
    const uint16_t *xrow[MT];
    const int8_t *qxrow[MT];
    bool col_ok[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int col = m0 + 16 * mt + r;
        col_ok[mt] = col < m;
        xrow[mt] = x + (int64_t)(col_ok[mt] ? col : 0) * k;
        qxrow[mt] = static_cast<const int8_t *>(xv) + (int64_t)(col_ok[mt] ? col : 0) * k;
    }

    // the scales of the outputs this lane ends up holding (channels
    // n0 + 16 t + 4 g + i), loaded now so that they arrive during the main
    // loop instead of stalling the epilogue
    uint16_t sc[RT][4];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int yn = n0 + 16 * t + 4 * g + i;
            sc[t][i] = yn < n ? scales[yn] : (uint16_t)0;
        }

    // asymmetric weights: the cast subtracts the zero point of weight row
    // n0 + 16 t + r (zeros == nullptr: symmetric)
    // (a template parameter: the symmetric kernels keep the constant bias
    // and its registers free)
    half2_t zbias[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t)
        zbias[t] = zero_point_bias(ZP && row_ok[t] ? (int)zeros[n0 + 16 * t + r] : 0);

    acc_t acc[RT][MT];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            acc[t][mt] = (acc_t){};

    for (int s = s_begin; s < s_end; s += kSkinnyUnroll) {
        u32x4_t wv[kSkinnyUnroll][RT];
        u32x4_t xa[kSkinnyUnroll][MT], xb[kSkinnyUnroll][MT];
        // Activation operands.  For the fp16 kernel with one activation
        // tile they are requested before the weight codes, so the two
        // loads' latencies overlap (measured 2-4% faster); otherwise after
        // the weight staging (two tiles measured 5% slower the other way,
        // and the int8 kernel kept its operand arrays in scratch memory).
        constexpr bool kXFirst = MT == 1 && !A8;
        if constexpr (kXFirst) {
#pragma unroll
            for (int u = 0; u < kSkinnyUnroll; ++u) {
                const int kk = (s + u) * 64 + g * 16;
                const bool ok = (s + u) < s_end && kk < k;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    xa[u][mt] = (u32x4_t){0u, 0u, 0u, 0u};
                    xb[u][mt] = (u32x4_t){0u, 0u, 0u, 0u};
                    if (ok && col_ok[mt]) {
                        if constexpr (A8) {
                            xa[u][mt] = *reinterpret_cast<const u32x4_t *>(qxrow[mt] + kk);
                        } else {
                            xa[u][mt] = *reinterpret_cast<const u32x4_t *>(xrow[mt] + kk);
                            xb[u][mt] = *reinterpret_cast<const u32x4_t *>(xrow[mt] + kk + 8);
                        }
                    }
                }
            }
        }
        {
            // Weight codes, loaded contiguously: instruction i of tile t
            // covers rows 4 i .. 4 i + 3, 256 bytes each (lane l: row
            // 4 i + l / 16, bytes 16 (l % 16) of the 256), so every load
            // instruction touches four 256-byte row segments instead of
            // sixteen 64-byte ones.  They go through this wave's slice of
            // LDS and come back in the MFMA layout (lane (r, g): row r,
            // bytes 64 u + 16 g for step u).
            uint8_t *slice = smem + wave * RT * 16 * kStageRow;
            const int ul = (lane % 16) / 4; // step this lane's 16 bytes belong to
            const int kl = s * 64 + 16 * (lane % 16);
            const bool okl = (s + ul) < s_end && kl < k;
            u32x4_t raw[4][RT];
#pragma unroll
            for (int t = 0; t < RT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = n0 + 16 * t + 4 * i + lane / 16;
                    raw[i][t] = (u32x4_t){0u, 0u, 0u, 0u};
                    if (okl && row < n)
                        raw[i][t] = __builtin_nontemporal_load(
                            reinterpret_cast<const u32x4_t *>(q + (int64_t)row * k + kl));
                }
#pragma unroll
            for (int t = 0; t < RT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<u32x4_t *>(slice + (t * 16 + 4 * i + lane / 16) * kStageRow +
                                                 16 * (lane % 16)) = raw[i][t];
            // Each lane reads back bytes that other lanes of the wave wrote.
            // LDS executes a wave's accesses in order, but per lane the read
            // and write addresses never coincide, so without these barriers
            // the compiler may move reads above the writes they depend on
            // (or the next iteration's writes above these reads).
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int u = 0; u < kSkinnyUnroll; ++u)
#pragma unroll
                for (int t = 0; t < RT; ++t)
                    wv[u][t] = *reinterpret_cast<const u32x4_t *>(slice + (t * 16 + r) * kStageRow + 64 * u + 16 * g);
            __builtin_amdgcn_wave_barrier();
        }
        if constexpr (!kXFirst) {
#pragma unroll
            for (int u = 0; u < kSkinnyUnroll; ++u) {
                const int kk = (s + u) * 64 + g * 16;
                const bool ok = (s + u) < s_end && kk < k;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    xa[u][mt] = (u32x4_t){0u, 0u, 0u, 0u};
                    xb[u][mt] = (u32x4_t){0u, 0u, 0u, 0u};
                    if (ok && col_ok[mt]) {
                        if constexpr (A8) {
                            xa[u][mt] = *reinterpret_cast<const u32x4_t *>(qxrow[mt] + kk);
                        } else {
                            xa[u][mt] = *reinterpret_cast<const u32x4_t *>(xrow[mt] + kk);
                            xb[u][mt] = *reinterpret_cast<const u32x4_t *>(xrow[mt] + kk + 8);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kSkinnyUnroll; ++u) {
            if constexpr (A8) {
#pragma unroll
                for (int t = 0; t < RT; ++t)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        acc[t][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                            __builtin_bit_cast(int4v, wv[u][t]), __builtin_bit_cast(int4v, xa[u][mt]), acc[t][mt],
                            0, 0, 0);
            } else {
#pragma unroll
                for (int t = 0; t < RT; ++t) {
                    const half8_t a0 = i8x8_to_half8(wv[u][t].x, wv[u][t].y, zbias[t]);
                    const half8_t a1 = i8x8_to_half8(wv[u][t].z, wv[u][t].w, zbias[t]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const half8_t b0 = __builtin_bit_cast(half8_t, xa[u][mt]);
                        const half8_t b1 = __builtin_bit_cast(half8_t, xb[u][mt]);
                        acc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b0, acc[t][mt], 0, 0, 0);
                        acc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b1, acc[t][mt], 0, 0, 0);
                    }
                }
            }
        }
    }

    if (KSPLIT > 1) {
        acc_t *partial = reinterpret_cast<acc_t *>(smem); // [KSPLIT-1][RT][MT][kWave]
        __syncthreads(); // every wave is done with its staging slice
        if (wave > 0) {
#pragma unroll
            for (int t = 0; t < RT; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    partial[(((wave - 1) * RT + t) * MT + mt) * kWave + lane] = acc[t][mt];
        }
        __syncthreads();
        if (wave != 0)
            return;
#pragma unroll
        for (int w = 0; w < KSPLIT - 1; ++w)
#pragma unroll
            for (int t = 0; t < RT; ++t)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[t][mt] += partial[((w * RT + t) * MT + mt) * kWave + lane];
    }
    // lane holds channels n0 + 16 t + 4 g + i (i = 0..3) of activation row
    // m0 + 16 mt + r: scale, round, and transpose through LDS so that the
    // stores are whole 16-byte pieces of Y rows
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const float xscale = A8 && col_ok[mt] ? f16_bits_to_f32(sx[m0 + 16 * mt + r]) : 0.0f;
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float out;
                if constexpr (A8) // exact int32 sum, then S[n] * Sx[m] (exact in fp32)
                    out = (float)acc[t][mt][i] * (f16_bits_to_f32(sc[t][i]) * xscale);
                else
                    out = acc[t][mt][i] * f16_bits_to_f32(sc[t][i]);
                // exact outliers of channel n0 + 16 t + 4 g + i, with X read
                // from global memory (a few activation rows: L2-resident)
                const int yn = n0 + 16 * t + 4 * g + i;
                if (!A8 && ol.idx != nullptr && yn < n && col_ok[mt]) {
                    for (int e = 0; e < ol.cap; ++e) {
                        const int kk = ol.idx[(int64_t)yn * ol.cap + e];
                        if (kk < 0 || kk >= k)
                            break; // used slots come first
                        out += f16_bits_to_f32(xrow[mt][kk]) * ol.val[(int64_t)yn * ol.cap + e];
                    }
                }
                ytile[16 * mt + r][16 * t + 4 * g + i] = f32_to_f16_bits(out);
            }
    }
    // the tile is written and read back by the same wave: LDS keeps a
    // wave's accesses in order; the barrier only stops the compiler from
    // moving the reads above the writes
    __builtin_amdgcn_wave_barrier();
    constexpr int kPieces = 16 * RT / 8;  // 16-byte pieces per tile row
    const bool vec_ok = (n % 8) == 0 && n0 + 16 * RT <= n;
    for (int e = lane; e < 16 * MT * kPieces; e += kWave) {
        const int row = e / kPieces;
        const int pc = e % kPieces;
        const int ym = m0 + row;
        if (ym >= m)
            continue;
        uint16_t *dst = y + (int64_t)ym * n + n0 + 8 * pc;
        if (vec_ok) {
            *reinterpret_cast<u32x4_t *>(dst) = *reinterpret_cast<const u32x4_t *>(&ytile[row][8 * pc]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (n0 + 8 * pc + j < n)
                    dst[j] = ytile[row][8 * pc + j];
        }
    }
}

template <int RT, int MT, int KSPLIT, bool A8>
hipError_t launch_cfg(const void *x, const uint16_t *sx, const int8_t *q, const uint16_t *scales,
                      const int8_t *zeros, OutlierList ol, uint16_t *y, int64_t m, int64_t n, int64_t k,
                      hipStream_t stream)
{
    const dim3 grid((unsigned)((n + 16 * RT - 1) / (16 * RT)), (unsigned)((m + 16 * MT - 1) / (16 * MT)));
    if constexpr (!A8) {
        if (zeros != nullptr) {
            hipLaunchKernelGGL((skinny_gemm_kernel<RT, MT, KSPLIT, false, true>), grid, dim3(KSPLIT * kWave), 0,
                               stream, x, sx, q, scales, zeros, ol, y, (int)m, (int)n, (int)k);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((skinny_gemm_kernel<RT, MT, KSPLIT, A8>), grid, dim3(KSPLIT * kWave), 0, stream,
                       x, sx, q, scales, zeros, ol, y, (int)m, (int)n, (int)k);
    return hipGetLastError();
}

// Largest k split per kernel variant: a workgroup of 16 waves leaves each
// lane 128 registers, which the int8 kernel and the two-tile fp16 kernel
// exceed (they spilled); they stop at 8 waves.  Four weight tiles with two
// activation tiles stop at 4: at 8 they spilled, and their staging slices
// would fill most of the LDS.
template <int RT, int MT, bool A8>
constexpr int max_split()
{
    return RT == 4 ? 4 : (A8 || MT > 1) ? 8 : 16;
}

template <int RT, int MT, bool A8>
hipError_t launch_mt(const void *x, const uint16_t *sx, const int8_t *q, const uint16_t *scales,
                     const int8_t *zeros, OutlierList ol, uint16_t *y, int64_t m, int64_t n, int64_t k,
                     hipStream_t stream)
{
    // split k until the grid holds about kSkinnyTargetWaves waves, keeping
    // at least one 64-wide step per wave
    const int64_t tiles = ((n + 16 * RT - 1) / (16 * RT)) * ((m + 16 * MT - 1) / (16 * MT));
    const int64_t steps = (k + 63) / 64;
    constexpr int kMaxSplit = max_split<RT, MT, A8>();
    int ksplit = 1;
    while (ksplit < kMaxSplit && tiles * ksplit < kSkinnyTargetWaves && steps >= 2 * ksplit)
        ksplit *= 2;
    if (ksplit == 1)
        return launch_cfg<RT, MT, 1, A8>(x, sx, q, scales, zeros, ol, y, m, n, k, stream);
    if (ksplit == 2)
        return launch_cfg<RT, MT, 2, A8>(x, sx, q, scales, zeros, ol, y, m, n, k, stream);
    if (ksplit == 4)
        return launch_cfg<RT, MT, 4, A8>(x, sx, q, scales, zeros, ol, y, m, n, k, stream);
    if constexpr (kMaxSplit >= 8)
        if (ksplit == 8)
            return launch_cfg<RT, MT, 8, A8>(x, sx, q, scales, zeros, ol, y, m, n, k, stream);
    if constexpr (kMaxSplit >= 16)
        if (ksplit == 16)
            return launch_cfg<RT, MT, 16, A8>(x, sx, q, scales, zeros, ol, y, m, n, k, stream);
    return hipErrorInvalidValue; // not reached: ksplit <= kMaxSplit
}

// Activation tiles per wave from m and k.  For 17..32 rows with k >= 2048,
// two tiles per wave take one pass over the weights instead of two
// (measured 10% faster at k = 4096, n = 4608 and 27392).  Otherwise one
// tile per wave and one pass per 16 rows: the passes run side by side and
// their repeated weight reads hit in cache, so more, shorter waves win
// (four tiles per wave measured 7-10% slower than four passes at 48 and 64
// rows; two tiles 2-5% slower at k = 1024, where the k split then has too
// few steps to fill the chip).
template <int RT, bool A8>
hipError_t launch_rt(const void *x, const uint16_t *sx, const int8_t *q, const uint16_t *scales,
                     const int8_t *zeros, OutlierList ol, uint16_t *y, int64_t m, int64_t n, int64_t k,
                     hipStream_t stream)
{
    if (skinny_rows_per_pass(m, k) == 32)
        return launch_mt<RT, 2, A8>(x, sx, q, scales, zeros, ol, y, m, n, k, stream);
    return launch_mt<RT, 1, A8>(x, sx, q, scales, zeros, ol, y, m, n, k, stream);
}

} // namespace

int skinny_rows_per_pass(int64_t m, int64_t k)
{
    return (m > 16 && m <= 32 && k >= 2048) ? 32 : 16;
}

namespace {

// Weight tiles per workgroup.  Two 16-row tiles share each activation
// operand load, but each workgroup holds all the k-split waves of its tiles,
// so the grid has one workgroup per RT x 16 weight rows (per pass).  Where
// one tile per workgroup still fits the grid on the chip in one round, the
// doubled workgroup count keeps twice the CUs streaming: at n = 4096, m = 8
// it measured 24% faster at k = 1024 and 12% at k = 4096 (128 two-tile
// workgroups leave half the CUs idle).  At n = 4608 (288 one-tile
// workgroups, a second round) two tiles stay faster.
template <bool A8>
hipError_t launch_auto_rt(const void *x, const uint16_t *sx, const int8_t *q, const uint16_t *scales,
                          const int8_t *zeros, OutlierList ol, uint16_t *y, int64_t m, int64_t n, int64_t k,
                          hipStream_t stream)
{
    const int64_t rows = skinny_rows_per_pass(m, k);
    const int64_t one_tile_grid = ((n + 15) / 16) * ((m + rows - 1) / rows);
    if (one_tile_grid <= device_cu_count())
        return launch_rt<1, A8>(x, sx, q, scales, zeros, ol, y, m, n, k, stream);
    // Two activation tiles read 32 activation rows per k step, once per
    // workgroup: four weight tiles halve those reads where the grid stays
    // large (n >= 12288 at one pass).  Measured at k = 4096: 49.4 -> 37.0 us
    // at m = 32 and n = 27392, 31.8 -> 26.7 us at m = 32 and n = 13824,
    // W8A8 m = 32, n = 27392 33.9 -> 28.1 us.  With one activation tile
    // four tiles measured slower on some of these grids.
    if (rows == 32 && one_tile_grid >= 3 * (int64_t)device_cu_count())
        return launch_mt<4, 2, A8>(x, sx, q, scales, zeros, ol, y, m, n, k, stream);
    return launch_rt<2, A8>(x, sx, q, scales, zeros, ol, y, m, n, k, stream);
}

} // namespace

hipError_t launch_skinny_gemm(const uint16_t *x, const int8_t *q, const uint16_t *scales,
                              const int8_t *zeros, OutlierList ol, uint16_t *y, int64_t m, int64_t n, int64_t k, hipStream_t stream)
{
    // one, two or four 16-row weight tiles per wave (more tiles reuse the
    // activation operand; four only with two activation tiles on a large
    // grid, elsewhere they measured slower: fewer waves, longer dependent
    // MFMA chains)
    return launch_auto_rt<false>(x, nullptr, q, scales, zeros, ol, y, m, n, k, stream);
}

hipError_t launch_w8a8_skinny(const int8_t *qx, const uint16_t *sx, const int8_t *q, const uint16_t *scales,
                              uint16_t *y, int64_t m, int64_t n, int64_t k, hipStream_t stream)
{
    return launch_auto_rt<true>(qx, sx, q, scales, nullptr, OutlierList{nullptr, nullptr, 0}, y, m, n, k, stream);
}

} // namespace qw

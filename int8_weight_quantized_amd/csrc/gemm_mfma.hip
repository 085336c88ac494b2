// gemm_mfma.hip -- W8A16 prefill GEMM on the matrix cores (gfx950).
//
// Prefill multiplies max_length activation rows with every weight, so the
// matmul itself dominates ("探索ChatGLM2在算能BM1684X上INT8量化部署",
// section 4: the W8A16 gain shrinks as max_length grows).  Each workgroup
// computes a BN x BM tile of Y^T (BN output channels x BM activation rows)
// with v_mfma_f32_16x16x32_f16 and fp32 accumulators; the per-channel
// scale multiplies the accumulators in the epilogue, which rounds to fp16
// and stores.
//
// Operands.  The MFMA "A" operand is the weight (rows = output channels),
// "B" the activations (columns = activation rows), so every lane ends up
// with 4 consecutive output channels of one activation row and stores 8
// contiguous bytes of Y.  The weight tile stays int8 in LDS (half the bytes
// of fp16 through LDS) and is cast to fp16 exactly in registers right
// after the LDS read; the cast runs on the VALU alongside the MFMAs.
//
// k assignment.  One k step is 64 wide.  Lane l (r = l % 16, g = l / 16)
// reads 16 codes [16 g, 16 g + 16) of weight row r: codes 0-7 feed one
// MFMA, codes 8-15 a second one, and the activation operand of lane l is
// read at the same k positions, so each MFMA contracts exactly the 32 k
// values its two operands agree on.
//
// Pipeline.  256 threads = 2 x 2 waves, each owning a (BN/2) x (BM/2)
// sub-tile (acc in AGPRs).  The next k tile is loaded from global memory
// into registers before the current tile's MFMAs are issued, then copied
// into the other half of a double-buffered LDS; one barrier per k step.
// LDS rows are padded by 16 bytes so that the 16 lanes reading one 16-byte
// column slice of 16 consecutive rows hit distinct banks.
//
// Grid.  Workgroups are renumbered so that each XCD (dispatch is
// round-robin over the 8 XCDs) walks a contiguous run of tiles; the
// activation tiles of one weight tile are consecutive, so the weight tile
// is reused from that XCD's L2.
#include "qw_device.h"
#include "qw_internal.h"

namespace qw {
namespace {

typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kGemmThreads = 256; // 2 x 2 waves
constexpr int kBK = 64;            // k per step
constexpr int kWRow = kBK + 16;    // LDS bytes per int8 weight row (padded)
constexpr int kXRow = 2 * kBK + 16; // LDS bytes per fp16 activation row (padded)

template <int BN, int BM>
struct TileCfg {
    static constexpr int kWaveN = BN / 2; // output channels per wave
    static constexpr int kWaveM = BM / 2; // activation rows per wave
    static constexpr int kSubN = kWaveN / 16;
    static constexpr int kSubM = kWaveM / 16;
    static constexpr int kWChunks = BN * kBK / 16;     // 16-byte chunks of the int8 W tile
    static constexpr int kXChunks = BM * kBK * 2 / 16; // 16-byte chunks of the fp16 X tile
    static constexpr int kWPerThread = kWChunks / kGemmThreads;
    static constexpr int kXPerThread = kXChunks / kGemmThreads;
    static constexpr int kWBytes = BN * kWRow;
    static constexpr int kXBytes = BM * kXRow;
    static constexpr int kStageBytes = kWBytes + kXBytes;
    static_assert(kWChunks % kGemmThreads == 0 && kXChunks % kGemmThreads == 0, "tile/thread mismatch");
    static_assert(kSubN >= 1 && kSubM >= 1, "wave tile below one MFMA tile");
};

__device__ __forceinline__ int xcd_remap(int bid, int nblocks)
{
    const int per = nblocks / 8, rem = nblocks % 8;
    const int xcd = bid % 8, local = bid / 8;
    return xcd * per + (xcd < rem ? xcd : rem) + local;
}

template <int BN, int BM>
__global__ __launch_bounds__(kGemmThreads) void mfma_gemm_kernel(
    const uint16_t *__restrict__ x, const int8_t *__restrict__ q,
    const uint16_t *__restrict__ scales, uint16_t *__restrict__ y,
    int m, int n, int k, int tiles_m, int tiles_n)
{
    using C = TileCfg<BN, BM>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * C::kStageBytes];

    const int tid = threadIdx.x;
    const int lane = __lane_id();
    const int wave = tid / kWave;
    const int wave_n = wave % 2;
    const int wave_m = wave / 2;

    const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    const int tn = tile / tiles_m;
    const int tm = tile % tiles_m;
    const int n0 = tn * BN;
    const int m0 = tm * BM;
    const int ktiles = (k + kBK - 1) / kBK;

    u32x4_t wreg[C::kWPerThread];
    u32x4_t xreg[C::kXPerThread];

    auto load_tile = [&](int kt) {
        const int k0 = kt * kBK;
#pragma unroll
        for (int i = 0; i < C::kWPerThread; ++i) {
            const int c = tid + i * kGemmThreads;
            const int row = c / (kBK / 16);
            const int kc = c % (kBK / 16);
            const int gn = n0 + row;
            const int gk = k0 + kc * 16;
            wreg[i] = (u32x4_t){0u, 0u, 0u, 0u};
            if (gn < n && gk < k)
                wreg[i] = *reinterpret_cast<const u32x4_t *>(q + (int64_t)gn * k + gk);
        }
#pragma unroll
        for (int i = 0; i < C::kXPerThread; ++i) {
            const int c = tid + i * kGemmThreads;
            const int row = c / (kBK / 8);
            const int kc = c % (kBK / 8);
            const int gm = m0 + row;
            const int gk = k0 + kc * 8;
            xreg[i] = (u32x4_t){0u, 0u, 0u, 0u};
            if (gm < m && gk < k)
                xreg[i] = *reinterpret_cast<const u32x4_t *>(x + (int64_t)gm * k + gk);
        }
    };

    auto store_tile = [&](int buf) {
        uint8_t *ws = lds + buf * C::kStageBytes;
        uint8_t *xs = ws + C::kWBytes;
#pragma unroll
        for (int i = 0; i < C::kWPerThread; ++i) {
            const int c = tid + i * kGemmThreads;
            const int row = c / (kBK / 16);
            const int kc = c % (kBK / 16);
            *reinterpret_cast<u32x4_t *>(ws + row * kWRow + kc * 16) = wreg[i];
        }
#pragma unroll
        for (int i = 0; i < C::kXPerThread; ++i) {
            const int c = tid + i * kGemmThreads;
            const int row = c / (kBK / 8);
            const int kc = c % (kBK / 8);
            *reinterpret_cast<u32x4_t *>(xs + row * kXRow + kc * 16) = xreg[i];
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
        const uint8_t *ws = lds + buf * C::kStageBytes;
        const uint8_t *xs = ws + C::kWBytes;

        half8_t b0[C::kSubM], b1[C::kSubM];
#pragma unroll
        for (int j = 0; j < C::kSubM; ++j) {
            const uint8_t *p = xs + (wave_m * C::kWaveM + j * 16 + lrow) * kXRow + lgrp * 32;
            b0[j] = *reinterpret_cast<const half8_t *>(p);
            b1[j] = *reinterpret_cast<const half8_t *>(p + 16);
        }
#pragma unroll
        for (int i = 0; i < C::kSubN; ++i) {
            const u32x4_t codes = *reinterpret_cast<const u32x4_t *>(
                ws + (wave_n * C::kWaveN + i * 16 + lrow) * kWRow + lgrp * 16);
            const half8_t a0 = i8x8_to_half8(codes.x, codes.y);
            const half8_t a1 = i8x8_to_half8(codes.z, codes.w);
#pragma unroll
            for (int j = 0; j < C::kSubM; ++j) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b0[j], acc[i][j], 0, 0, 0);
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b1[j], acc[i][j], 0, 0, 0);
            }
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

template <int BN, int BM>
hipError_t launch_cfg(const uint16_t *x, const int8_t *q, const uint16_t *scales, uint16_t *y,
                      int64_t m, int64_t n, int64_t k, hipStream_t stream)
{
    const int64_t tiles_m = (m + BM - 1) / BM;
    const int64_t tiles_n = (n + BN - 1) / BN;
    const int64_t blocks = tiles_m * tiles_n;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((mfma_gemm_kernel<BN, BM>), dim3((unsigned)blocks), dim3(kGemmThreads), 0,
                       stream, x, q, scales, y, (int)m, (int)n, (int)k, (int)tiles_m, (int)tiles_n);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Big-tile variant for prefill-sized m: 256 x 256 output tile per
// workgroup, one wave per SIMD, each wave 128 x 128 (256 fp32 accumulators
// in AGPRs).  Operands are copied from global memory straight into LDS by
// the gfx950 LDS-DMA loads (global_load_lds_dwordx4: each lane's 16 bytes
// land at LDS base + 16 * lane) through a 3-stage ring:
//
//   iteration t:
//     wait for my copies of tile t; barrier (everyone's copies landed,
//       everyone done reading tile t-1)
//     start copying tile t+2 into tile t-1's stage
//     LDS -> registers: operands of tile t; MFMAs of tile t
//
// so up to two tiles are in flight while one is multiplied; one barrier
// per k step.  (Measured: prefetching the next tile's operands into a
// second register set during the MFMAs was slower here; the register
// copies it needs stall on MFMA source-operand hazards.)
//
// LDS-DMA writes 1 KiB contiguous per wave instruction, so rows cannot be
// padded; instead 16-byte chunks are XOR-swizzled within a row, with a
// pattern that depends on the row's position inside its aligned group of
// 16 (r16 = row % 16):
//   weight row (64 int8):       chunk c at slot c ^ (((r16 >> 1) ^ (r16 >> 3)) & 3)
//   activation row (64 fp16):   chunk c at slot c ^ ((r16 ^ (r16 >> 3)) & 7)
// With these, the 16 rows one 16-lane group reads (and any 8 of them) land
// in distinct banks.  The lane that fills a slot loads the matching
// logical chunk.  Rows beyond n or m load a clamped valid row (their
// outputs are never stored); k chunks beyond k are zero-filled with
// ordinary LDS stores.
// ---------------------------------------------------------------------------
constexpr int kDmaBN = 256, kDmaBM = 256;
constexpr int kDmaWBytes = kDmaBN * kBK;     // 16 KiB int8
constexpr int kDmaXBytes = kDmaBM * kBK * 2; // 32 KiB fp16
constexpr int kDmaStage = kDmaWBytes + kDmaXBytes;
constexpr int kDmaStages = 3;
constexpr int kDmaWInstr = kDmaWBytes / 1024 / 4; // per wave per stage
constexpr int kDmaXInstr = kDmaXBytes / 1024 / 4;
constexpr int kDmaInstr = kDmaWInstr + kDmaXInstr;
constexpr int kDmaSN = 8, kDmaSM = 8; // 16 x 16 MFMA tiles per wave

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
#define QW_WAIT_VMCNT(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (7 << 4) | (15 << 8) | (((N) >> 4) << 14))

__device__ __forceinline__ void wait_lgkmcnt0()
{
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Wait until at most `tiles` tiles' worth of this wave's copies are in
// flight (0, 1 or 2 tiles).
__device__ __forceinline__ void wait_tiles_in_flight(int tiles)
{
    if (tiles >= 2)
        QW_WAIT_VMCNT(2 * kDmaInstr);
    else if (tiles == 1)
        QW_WAIT_VMCNT(kDmaInstr);
    else
        QW_WAIT_VMCNT(0);
}

// Barrier without a memory fence: a workgroup fence would make the compiler
// drain every in-flight LDS-DMA copy (vmcnt(0)) and empty the ring.  The
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void ring_barrier()
{
    wait_lgkmcnt0();
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
}

__device__ __forceinline__ int wslot(int row)
{
    const int r16 = row & 15;
    return ((r16 >> 1) ^ (r16 >> 3)) & 3;
}

__device__ __forceinline__ int xslot(int row)
{
    const int r16 = row & 15;
    return (r16 ^ (r16 >> 3)) & 7;
}

struct DmaOperands {
    u32x4_t codes[kDmaSN];
    half8_t b0[kDmaSM];
};

__global__ __launch_bounds__(kGemmThreads) void mfma_gemm_dma_kernel(
    const uint16_t *__restrict__ x, const int8_t *__restrict__ q,
    const uint16_t *__restrict__ scales, uint16_t *__restrict__ y,
    int m, int n, int k, int tiles_m, int tiles_n)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kDmaStages * kDmaStage];

    const int tid = threadIdx.x;
    const int lane = __lane_id();
    const int wave = tid / kWave;
    const int wave_n = wave % 2;
    const int wave_m = wave / 2;

    const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    const int tn = tile / tiles_m;
    const int tm = tile % tiles_m;
    const int n0 = tn * kDmaBN;
    const int m0 = tm * kDmaBM;
    const int ktiles = (k + kBK - 1) / kBK;
    // the last tile issues fewer copies when k is ragged; waits then drain
    const int full_tiles = (k % kBK) != 0 ? ktiles - 1 : ktiles;

    // DMA source mapping.  Weight copy i of this wave covers tile rows
    // (wave * kDmaWInstr + i) * 16 + [0, 16): lane -> row + lane / 4, slot
    // lane % 4; activation copy i covers rows (wave * kDmaXInstr + i) * 8 +
    // [0, 8): lane -> row + lane / 8, slot lane % 8.  The logical chunk a
    // slot holds depends only on the row within its group of 16, so it is
    // the same for every weight copy and alternates for activation copies.
    const int wchunk = (lane % 4) ^ wslot(lane / 4);
    const int xchunk_even = (lane % 8) ^ xslot(lane / 8);
    const int xchunk_odd = (lane % 8) ^ xslot(8 + lane / 8);

    auto issue = [&](int kt) {
        uint8_t *st = lds + (kt % kDmaStages) * kDmaStage;
        const int k0 = kt * kBK;
#pragma unroll
        for (int i = 0; i < kDmaWInstr; ++i) {
            uint8_t *dst = st + (wave * kDmaWInstr + i) * 1024;
            const int row = (wave * kDmaWInstr + i) * 16 + lane / 4;
            const int gn = min(n0 + row, n - 1);
            const int gk = k0 + wchunk * 16;
            if (gk < k)
                __builtin_amdgcn_global_load_lds(q + (int64_t)gn * k + gk, (lds_ptr_t)dst, 16, 0, 0);
            else
                *reinterpret_cast<u32x4_t *>(dst + lane * 16) = (u32x4_t){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < kDmaXInstr; ++i) {
            uint8_t *dst = st + kDmaWBytes + (wave * kDmaXInstr + i) * 1024;
            const int row = (wave * kDmaXInstr + i) * 8 + lane / 8;
            const int gm = min(m0 + row, m - 1);
            const int gk = k0 + ((i & 1) ? xchunk_odd : xchunk_even) * 8;
            if (gk < k)
                __builtin_amdgcn_global_load_lds(x + (int64_t)gm * k + gk, (lds_ptr_t)dst, 16, 0, 0);
            else
                *reinterpret_cast<u32x4_t *>(dst + lane * 16) = (u32x4_t){0u, 0u, 0u, 0u};
        }
    };
    // copies still in flight behind tile t when tile t is waited for (tile
    // t+1 if it exists); a ragged tail tile may issue fewer copies, so a
    // wait that would leave it outstanding drains completely instead
    auto tiles_behind = [&](int t) {
        const int last_issued = min(t + 1, ktiles - 1);
        const int behind = last_issued - t;
        return last_issued >= full_tiles ? 0 : behind;
    };

    const int lrow = lane % 16;
    const int lgrp = lane / 16;
    // this lane's operand slices inside a stage (rows base + 16 i + lrow)
    const int wrow = wave_n * 128 + lrow;
    const int w_off = wrow * kBK + 16 * (lgrp ^ wslot(wrow));
    const int xrow = wave_m * 128 + lrow;
    const int x_off0 = kDmaWBytes + xrow * 2 * kBK + 16 * ((2 * lgrp) ^ xslot(xrow));
    const int x_off1 = kDmaWBytes + xrow * 2 * kBK + 16 * ((2 * lgrp + 1) ^ xslot(xrow));

    // codes (both k halves) and first-half activations of tile kt
    auto read_operands = [&](int kt, DmaOperands &op) {
        const uint8_t *st = lds + (kt % kDmaStages) * kDmaStage;
#pragma unroll
        for (int i = 0; i < kDmaSN; ++i)
            op.codes[i] = *reinterpret_cast<const u32x4_t *>(st + w_off + i * 16 * kBK);
#pragma unroll
        for (int j = 0; j < kDmaSM; ++j)
            op.b0[j] = *reinterpret_cast<const half8_t *>(st + x_off0 + j * 16 * 2 * kBK);
    };
    // second-half activations of tile kt
    auto read_b1 = [&](int kt, half8_t (&b1)[kDmaSM]) {
        const uint8_t *st = lds + (kt % kDmaStages) * kDmaStage;
#pragma unroll
        for (int j = 0; j < kDmaSM; ++j)
            b1[j] = *reinterpret_cast<const half8_t *>(st + x_off1 + j * 16 * 2 * kBK);
    };

    float4v acc[kDmaSN][kDmaSM];
#pragma unroll
    for (int i = 0; i < kDmaSN; ++i)
#pragma unroll
        for (int j = 0; j < kDmaSM; ++j)
            acc[i][j] = (float4v){0.f, 0.f, 0.f, 0.f};

    // prologue: two tiles in flight
    issue(0);
    if (ktiles > 1)
        issue(1);

    for (int t = 0; t < ktiles; ++t) {
        // my copies of tile t are done once at most one tile's copies remain
        // outstanding; then the barrier publishes everyone's copies and
        // certifies that the stage tile t+2 goes to (tile t-1's) is no
        // longer being read
        wait_tiles_in_flight(tiles_behind(t) > 0 ? 1 : 0);
        ring_barrier();
        if (t + 2 < ktiles)
            issue(t + 2);

        DmaOperands op;
        half8_t b1[kDmaSM];
        read_operands(t, op);
        read_b1(t, b1);
        half8_t a0 = i8x8_to_half8(op.codes[0].x, op.codes[0].y);
        half8_t a1 = i8x8_to_half8(op.codes[0].z, op.codes[0].w);
#pragma unroll
        for (int i = 0; i < kDmaSN; ++i) {
            // cast the next weight sub-tile while this one's MFMAs run
            half8_t n0v = a0, n1v = a1;
            if (i + 1 < kDmaSN) {
                n0v = i8x8_to_half8(op.codes[i + 1].x, op.codes[i + 1].y);
                n1v = i8x8_to_half8(op.codes[i + 1].z, op.codes[i + 1].w);
            }
#pragma unroll
            for (int j = 0; j < kDmaSM; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, op.b0[j], acc[i][j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < kDmaSM; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b1[j], acc[i][j], 0, 0, 0);
            a0 = n0v;
            a1 = n1v;
        }
    }

    // ---- epilogue: scale, round to fp16, store ----
    const bool vec_ok = (n % 4) == 0;
#pragma unroll
    for (int i = 0; i < kDmaSN; ++i) {
        const int gn = n0 + wave_n * 128 + i * 16 + lgrp * 4;
        float s[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            s[r] = (gn + r < n) ? f16_bits_to_f32(scales[gn + r]) : 0.0f;
#pragma unroll
        for (int j = 0; j < kDmaSM; ++j) {
            const int gm = m0 + wave_m * 128 + j * 16 + lrow;
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

hipError_t launch_dma(const uint16_t *x, const int8_t *q, const uint16_t *scales, uint16_t *y,
                      int64_t m, int64_t n, int64_t k, hipStream_t stream)
{
    const int64_t tiles_m = (m + kDmaBM - 1) / kDmaBM;
    const int64_t tiles_n = (n + kDmaBN - 1) / kDmaBN;
    const int64_t blocks = tiles_m * tiles_n;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(mfma_gemm_dma_kernel, dim3((unsigned)blocks), dim3(kGemmThreads), 0, stream,
                       x, q, scales, y, (int)m, (int)n, (int)k, (int)tiles_m, (int)tiles_n);
    return hipGetLastError();
}

} // namespace

hipError_t launch_mfma_gemm(const uint16_t *x, const int8_t *q, const uint16_t *scales, uint16_t *y,
                            int64_t m, int64_t n, int64_t k, hipStream_t stream)
{
    if (m <= 32)
        return launch_cfg<128, 32>(x, q, scales, y, m, n, k, stream);
    if (m <= 64)
        return launch_cfg<128, 64>(x, q, scales, y, m, n, k, stream);
    if (m <= 128)
        return launch_cfg<256, 128>(x, q, scales, y, m, n, k, stream);
    return launch_dma(x, q, scales, y, m, n, k, stream);
}

} // namespace qw

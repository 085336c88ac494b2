// gemm_mfma.hip -- W8A16 GEMM on the matrix cores (gfx950), for prefill and
// other activation counts beyond the skinny kernel's range.
//
// Prefill multiplies max_length activation rows with every weight, so the
// matmul itself dominates ("探索ChatGLM2在算能BM1684X上INT8量化部署",
// section 4: the W8A16 gain shrinks as max_length grows).  Each workgroup
// computes a BN x BM tile of Y^T (BN output channels x BM activation rows)
// with v_mfma_f32_32x32x16_f16 and fp32 accumulators; the per-channel scale
// multiplies the accumulators in the epilogue, which rounds to fp16 and
// stores.  The weight is the MFMA "A" operand (rows = output channels), the
// activations the "B" operand (columns = activation rows).  The weight tile
// stays int8 in LDS (half the bytes of fp16 through LDS) and is cast to fp16
// exactly in registers right after the LDS read.
//
// Tile shapes.  BN x BM in {256 x 128, 256 x 64, 128 x 128, 128 x 64}: the
// launcher takes the largest tile whose grid still fills three quarters of
// the workgroup slots the chip holds at once (a tile's slot count is its
// occupancy per CU times the CU count), else the smallest.  Measured on
// MI355X: 256 x 128 for 512 x 4096 x 27392 and 4096 x 1024 x 4096, 128 x 128
// for 256 rows, 128 x 64 for up to ~100 rows or narrow weights (N = 4608)
// where larger tiles leave most CUs idle.
//
// Grid.  Workgroups are renumbered so that each XCD (dispatch is
// round-robin over the 8 XCDs) walks a contiguous run of tiles.  Along
// that run the tiles go in groups of `group` weight-tile columns, the
// activation tiles walking down each group, so the tiles an XCD holds at
// once form a near-square block: each weight and activation k-slice is
// fetched into that XCD's L2 once for the whole block.
#include "qw_device.h"
#include "qw_internal.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <type_traits>

namespace qw {
namespace {

typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int2v __attribute__((ext_vector_type(2)));
typedef int int16v __attribute__((ext_vector_type(16)));

constexpr int kBK = 64; // k per step

template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

__device__ __forceinline__ int xcd_remap(int bid, int nblocks)
{
    const int per = nblocks / 8, rem = nblocks % 8;
    const int xcd = bid % 8, local = bid / 8;
    return xcd * per + (xcd < rem ? xcd : rem) + local;
}

// ---------------------------------------------------------------------------
// Big-tile variant for prefill-sized m: a BN x BM output tile per
// workgroup of 4 waves (one per SIMD), each wave BN / 4 output channels x
// all BM activation rows on v_mfma_f32_32x32x16_f16 with fp32 accumulators
// in registers.  (Splitting the channels rather than the rows halves the
// per-wave int8 -> fp16 casts, each cast weight operand feeding BM / 32
// MFMAs; the price is that every wave reads the whole activation tile.)
// Operands are copied from global memory straight into LDS by the gfx950
// LDS-DMA loads (buffer_load_dwordx4 ... lds in full k steps,
// global_load_lds_dwordx4 in the ragged last ones: each lane's 16 bytes
// land at LDS base + 16 * lane) into two LDS stages:
//
//   step t:
//     wait for my copies of tile t; barrier (everyone's copies landed,
//       everyone done reading tile t-1)
//     start copying tile t + 1 into tile t-1's stage (on the 256-channel
//       fp16 tiles, spread over the step's four MFMA groups)
//     LDS -> registers: operands of tile t; dequantize; MFMAs of tile t
//
// one barrier per k step.  (Two workgroups of 67 KiB share a CU, so the
// second one's MFMAs fill the first one's copy and LDS phases; a third
// stage would not fit twice.)  Each stage is a separate LDS array and the
// steady-state loop is unrolled by two so that every access names its
// array at compile time: the compiler then sees that the LDS reads of
// tile t cannot alias the copies in flight into other stages and does not
// wait for them (with one array it drains every copy before the first LDS
// read of each step, which exposes the full copy latency per k step).
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

// NW waves per workgroup side by side along n; each wave owns BN / NW
// output channels x all BM activation rows.  A8: the activations are int8
// codes (W8A8) instead of fp16.
template <int NW, int BN, int BM, bool A8>
struct DmaCfg {
    static constexpr int kBN = BN;                            // output channels per workgroup
    static constexpr int kWBytes = BN * kBK;                  // int8 weight tile per stage
    static constexpr int kThreads = NW * kWave;
    static constexpr int kXBytes = BM * kBK * (A8 ? 1 : 2);  // activation tile per stage
    static constexpr int kStage = kWBytes + kXBytes;
    static constexpr int kWInstr = kWBytes / 1024 / NW;      // copies per wave per stage
    static constexpr int kXInstr = kXBytes / 1024 / NW;
    static constexpr int kInstr = kWInstr + kXInstr;
    static constexpr int kWaveN = BN / NW;                   // output channels per wave
    static constexpr int kSI = kWaveN / 32;                   // 32 x 32 MFMA tiles along n
    static constexpr int kSJ = BM / 32;                       // 32 x 32 MFMA tiles along m
    // epilogue: the fp16 output tile, [BM][BN] with rows padded by 16
    // bytes; rows [0, BM/2) go to stage 0's array, [BM/2, BM) to stage 1's
    static constexpr int kYRow = BN * 2 + 16;
    static constexpr int kYHalf = (BM / 2) * kYRow;
    static constexpr int kStageAlloc = kStage > kYHalf ? kStage : kYHalf;
    static_assert(kWInstr * 64 * 16 * NW == kWBytes && kXInstr * 64 * 16 * NW == kXBytes, "copy split");
    static_assert(A8 || kXInstr % 2 == 0, "fp16 activation copies alternate between the two 8-row swizzle phases");
    static_assert(kSI >= 1 && kWaveN % 32 == 0 && BM % 64 == 0, "tile config");
};

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// Word 3 of a raw (untyped, unswizzled, stride 0) buffer descriptor on the
// CDNA family: data format 32 bits per element, every other field 0.
constexpr int kBufferFlags = 0x00020000;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
#define QW_WAIT_VMCNT(N) __builtin_amdgcn_s_waitcnt(((N) & 15) | (7 << 4) | (15 << 8) | (((N) >> 4) << 14))

__device__ __forceinline__ void wait_lgkmcnt0()
{
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
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

template <int I>
using stage_t = std::integral_constant<int, I>;

// A8 (W8A8): x holds int8 activation codes with one fp16 scale per row in
// sx; the MFMA is v_mfma_i32_32x32x32_i8 with exact int32 accumulators and
// the epilogue multiplies by S[n] * Sx[m].  Otherwise x is fp16 and sx is
// unused.  OL: exact outlier side lists (at most kMfmaOutlierSlots per
// weight row) are added to the accumulators after the main loop.
template <int NW, int BN, int BM, bool A8, bool OL = false, bool ZP = false>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(NW == 4 && BM > 128 ? 1 : 2))) void mfma_gemm_dma_kernel(
    const void *__restrict__ xv, const uint16_t *__restrict__ sx, const int8_t *__restrict__ q,
    const uint16_t *__restrict__ scales, const int8_t *__restrict__ zeros, OutlierList ol,
    uint16_t *__restrict__ y, int m, int n, int k, int tiles_m, int tiles_n, int group)
{
    using C = DmaCfg<NW, BN, BM, A8>;
    constexpr int kSJ = C::kSJ;
    const uint16_t *__restrict__ x = static_cast<const uint16_t *>(xv);
    const int8_t *__restrict__ qx = static_cast<const int8_t *>(xv);
    __shared__ __attribute__((aligned(1024))) uint8_t ring0[C::kStageAlloc];
    __shared__ __attribute__((aligned(1024))) uint8_t ring1[C::kStageAlloc];
    __shared__ __attribute__((aligned(16))) float scale_lds[BN];
    __shared__ __attribute__((aligned(16))) float xscale_lds[A8 ? BM : 1];
    // OL: the workgroup's side lists, (column, value / S as float bits) per
    // slot; unused slots hold column INT_MAX
    __shared__ __attribute__((aligned(16))) int2v ol_lds[OL ? BN * kMfmaOutlierSlots : 1];
    auto ring = [&](auto s) -> uint8_t * {
        if constexpr (decltype(s)::value == 0)
            return ring0;
        else
            return ring1;
    };

    const int tid = threadIdx.x;
    const int lane = __lane_id();
    // wave-uniform (an SGPR): LDS-DMA destinations derived from it are
    // scalar, so setting M0 needs no v_readfirstlane per copy
    const int wave = __builtin_amdgcn_readlane(tid / kWave, 0);

    const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    // group gi holds weight-tile columns [gi * group, gi * group + gw); the
    // last group may be narrower
    const int gsize = group * tiles_m;
    const int gi = tile / gsize;
    const int gl = tile - gi * gsize;
    const int gw = min(group, tiles_n - gi * group);
    const int tn = gi * group + gl % gw;
    const int tm = gl / gw;
    const int n0 = tn * BN;
    const int m0 = tm * BM;
    const int ktiles = (k + kBK - 1) / kBK;
    // the last tile issues fewer copies when k is ragged; waits then drain
    const int full_tiles = (k % kBK) != 0 ? ktiles - 1 : ktiles;

    // DMA source mapping.  Weight copy i of this wave covers tile rows
    // (wave * kWInstr + i) * 16 + [0, 16): lane -> row + lane / 4, slot
    // lane % 4; activation copy i covers rows (wave * kXInstr + i) * 8 +
    // [0, 8): lane -> row + lane / 8, slot lane % 8.  The logical chunk a
    // slot holds depends only on the row within its group of 16, so it is
    // the same for every weight copy and alternates for activation copies.
    const int wchunk = (lane % 4) ^ wslot(lane / 4);
    const int xchunk_even = (lane % 8) ^ xslot(lane / 8);
    const int xchunk_odd = (lane % 8) ^ xslot(8 + lane / 8);

    // Per-lane byte offsets of this wave's copies from the tile's first row
    // at k = 0 (row clamped to the matrix); each full step then adds only
    // the wave-uniform k0 to a scalar base, so the copies can use the
    // scalar-base plus 32-bit-offset address form instead of per-step
    // 64-bit address math.
    uint32_t woff[C::kWInstr], xoff[C::kXInstr];
#pragma unroll
    for (int i = 0; i < C::kWInstr; ++i) {
        const int row = (wave * C::kWInstr + i) * 16 + lane / 4;
        woff[i] = (uint32_t)((min(n0 + row, n - 1) - n0) * k + wchunk * 16);
    }
#pragma unroll
    for (int i = 0; i < C::kXInstr; ++i) {
        if constexpr (A8) {
            const int row = (wave * C::kXInstr + i) * 16 + lane / 4;
            xoff[i] = (uint32_t)((min(m0 + row, m - 1) - m0) * k + wchunk * 16);
        } else {
            const int row = (wave * C::kXInstr + i) * 8 + lane / 8;
            xoff[i] = (uint32_t)(((min(m0 + row, m - 1) - m0) * k + ((i & 1) ? xchunk_odd : xchunk_even) * 8) * 2);
        }
    }
    const int8_t *wtile = q + (int64_t)n0 * k;
    const uint8_t *xtile = static_cast<const uint8_t *>(xv) + (int64_t)m0 * k * (A8 ? 1 : 2);
    // Buffer resources over this workgroup's weight and activation rows, so
    // that a full step's copies take the lane's 32-bit offset in a VGPR and
    // the step's k offset in an SGPR: no per-copy address arithmetic.  The
    // byte range (an unsigned 32-bit field; k <= 2^23 keeps it within 2^31)
    // covers the tile's rows; every copy lies inside it.
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t *>(wtile), (short)0,
        static_cast<int>(static_cast<uint32_t>(min((int64_t)BN, (int64_t)(n - n0)) * k)), kBufferFlags);
    const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(xtile), (short)0,
        static_cast<int>(static_cast<uint32_t>(min((int64_t)BM, (int64_t)(m - m0)) * k * (A8 ? 1 : 2))),
        kBufferFlags);

    // Copies of a tile that lies wholly inside k, in four groups: group g
    // (0..3) is this wave's weight and activation copies i with i % 4 == g.
    auto issue_group = [&](int kt, uint8_t *st, int g) {
        const int k0 = kt * kBK;
#pragma unroll
        for (int i = 0; i < C::kWInstr; ++i) {
            if (i % 4 != g)
                continue;
            uint8_t *dst = st + (wave * C::kWInstr + i) * 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wrsrc, (lds_ptr_t)dst, 16, (int)woff[i], k0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < C::kXInstr; ++i) {
            if (i % 4 != g)
                continue;
            uint8_t *dst = st + C::kWBytes + (wave * C::kXInstr + i) * 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xrsrc, (lds_ptr_t)dst, 16, (int)xoff[i], k0 * (A8 ? 1 : 2), 0,
                                                     0);
        }
    };

    // copy tile kt into stage array st; FULL: every chunk lies inside k
    auto issue = [&](int kt, uint8_t *st, auto full) {
        const int k0 = kt * kBK;
        if constexpr (decltype(full)::value) {
#pragma unroll
            for (int g = 0; g < 4; ++g)
                issue_group(kt, st, g);
            return;
        }
#pragma unroll
        for (int i = 0; i < C::kWInstr; ++i) {
            uint8_t *dst = st + (wave * C::kWInstr + i) * 1024;
            const int row = (wave * C::kWInstr + i) * 16 + lane / 4;
            const int gn = min(n0 + row, n - 1);
            const int gk = k0 + wchunk * 16;
            if (decltype(full)::value || gk < k)
                __builtin_amdgcn_global_load_lds(q + (int64_t)gn * k + gk, (lds_ptr_t)dst, 16, 0, 0);
            else
                *reinterpret_cast<u32x4_t *>(dst + lane * 16) = (u32x4_t){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < C::kXInstr; ++i) {
            uint8_t *dst = st + C::kWBytes + (wave * C::kXInstr + i) * 1024;
            if constexpr (A8) {
                // int8 activation rows are laid out like weight rows
                const int row = (wave * C::kXInstr + i) * 16 + lane / 4;
                const int gm = min(m0 + row, m - 1);
                const int gk = k0 + wchunk * 16;
                if (decltype(full)::value || gk < k)
                    __builtin_amdgcn_global_load_lds(qx + (int64_t)gm * k + gk, (lds_ptr_t)dst, 16, 0, 0);
                else
                    *reinterpret_cast<u32x4_t *>(dst + lane * 16) = (u32x4_t){0u, 0u, 0u, 0u};
            } else {
                const int row = (wave * C::kXInstr + i) * 8 + lane / 8;
                const int gm = min(m0 + row, m - 1);
                const int gk = k0 + ((i & 1) ? xchunk_odd : xchunk_even) * 8;
                if (decltype(full)::value || gk < k)
                    __builtin_amdgcn_global_load_lds(x + (int64_t)gm * k + gk, (lds_ptr_t)dst, 16, 0, 0);
                else
                    *reinterpret_cast<u32x4_t *>(dst + lane * 16) = (u32x4_t){0u, 0u, 0u, 0u};
            }
        }
    };
    using full_t = std::integral_constant<bool, true>;
    using partial_t = std::integral_constant<bool, false>;

    // v_mfma_f32_32x32x16_f16: lane l feeds row (l % 32) of A (a weight row)
    // and column (l % 32) of B (an activation row), 8 k values each; lane
    // group g = l / 32 takes k slots [8 g, 8 g + 8).  One 64-wide k step is
    // four MFMAs s = 0..3; in MFMA s, group g covers k = 32 g + 8 s + [0, 8),
    // so a lane reads 32 consecutive codes (two 16-byte chunks) of its
    // weight row and 32 consecutive activations (four chunks) of its
    // activation row per step.
    const int lrow = lane % 32;
    const int lgrp = lane / 32;
    const int wrow = wave * C::kWaveN + lrow;   // + 32 i
    const int w_off0 = wrow * kBK + 16 * ((2 * lgrp) ^ wslot(wrow));
    const int w_off1 = wrow * kBK + 16 * ((2 * lgrp + 1) ^ wslot(wrow));
    const int xrow = lrow;                      // + 32 j
    int x_off[4];
#pragma unroll
    for (int sidx = 0; sidx < 4; ++sidx)
        x_off[sidx] = C::kWBytes + xrow * 2 * kBK + 16 * ((4 * lgrp + sidx) ^ xslot(xrow));

    // A8: v_mfma_i32_32x32x32_i8 takes 16 consecutive k codes per lane, and
    // a 64-wide k step is two MFMAs s = 0, 1; in MFMA s, lane group g covers
    // the 16 codes of chunk 2 g + s of its row, for the weight (A) and the
    // activation (B) operand alike, so every k is paired with itself.
    const int xa_off0 = C::kWBytes + xrow * kBK + 16 * ((2 * lgrp) ^ wslot(xrow));
    const int xa_off1 = C::kWBytes + xrow * kBK + 16 * ((2 * lgrp + 1) ^ wslot(xrow));

    using acc_t = std::conditional_t<A8, int16v, float16v>;
    acc_t acc[C::kSI][kSJ];
#pragma unroll
    for (int i = 0; i < C::kSI; ++i)
#pragma unroll
        for (int j = 0; j < kSJ; ++j)
            acc[i][j] = (acc_t){};

    // asymmetric weights (zeros non-null, fp16 activations only): the cast
    // subtracts the zero point of each of this lane's weight rows
    half2_t zbias[C::kSI];
#pragma unroll
    for (int i = 0; i < C::kSI; ++i) {
        const int zr = n0 + wrow + 32 * i;
        zbias[i] = zero_point_bias(ZP && zr < n ? (int)zeros[zr] : 0); // ZP: symmetric kernels keep the constant
    }

    auto compute_a8 = [&](const uint8_t *st) {
        u32x4_t clo[C::kSI], chi[C::kSI];
#pragma unroll
        for (int i = 0; i < C::kSI; ++i) {
            clo[i] = *reinterpret_cast<const u32x4_t *>(st + w_off0 + i * 32 * kBK);
            chi[i] = *reinterpret_cast<const u32x4_t *>(st + w_off1 + i * 32 * kBK);
        }
        u32x4_t blo[kSJ], bhi[kSJ];
#pragma unroll
        for (int j = 0; j < kSJ; ++j) {
            blo[j] = *reinterpret_cast<const u32x4_t *>(st + xa_off0 + j * 32 * kBK);
            bhi[j] = *reinterpret_cast<const u32x4_t *>(st + xa_off1 + j * 32 * kBK);
        }
#pragma unroll
        for (int i = 0; i < C::kSI; ++i)
#pragma unroll
            for (int j = 0; j < kSJ; ++j)
                if constexpr (A8)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                        __builtin_bit_cast(int4v, clo[i]), __builtin_bit_cast(int4v, blo[j]), acc[i][j], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < C::kSI; ++i)
#pragma unroll
            for (int j = 0; j < kSJ; ++j)
                if constexpr (A8)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                        __builtin_bit_cast(int4v, chi[i]), __builtin_bit_cast(int4v, bhi[j]), acc[i][j], 0, 0, 0);
    };

    // The 256-channel fp16 tiles spread a full step's copies over the step
    // (see step below).  Their activation operands are then read one MFMA
    // group ahead, so that the copies can sit between the groups without
    // all of them live at once.  The 128-channel tiles measured slower with
    // spread copies (3% on 128 x 128, 11% on 128 x 64) and keep them at the
    // top of the step.
    constexpr bool kSpreadTile = !A8 && BN == 256;

    // before_group(s) runs ahead of MFMA group s = 0..3 of the fp16 path
    auto compute = [&](const uint8_t *st, auto &&before_group) {
      if constexpr (A8) {
        compute_a8(st);
      } else {
        u32x4_t clo[C::kSI], chi[C::kSI];
#pragma unroll
        for (int i = 0; i < C::kSI; ++i) {
            clo[i] = *reinterpret_cast<const u32x4_t *>(st + w_off0 + i * 32 * kBK);
            chi[i] = *reinterpret_cast<const u32x4_t *>(st + w_off1 + i * 32 * kBK);
        }
        half8_t b[kSJ][4];
        auto load_b = [&](int sidx) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < kSJ; ++j)
                b[j][sidx] = *reinterpret_cast<const half8_t *>(st + x_off[sidx] + j * 32 * 2 * kBK);
        };
#pragma unroll
        for (int sidx = 0; sidx < (kSpreadTile ? 1 : 4); ++sidx)
            load_b(sidx);
#pragma unroll
        for (int sidx = 0; sidx < 4; ++sidx) {
            before_group(sidx);
            if (kSpreadTile && sidx + 1 < 4)
                load_b(sidx + 1);
#pragma unroll
            for (int i = 0; i < C::kSI; ++i) {
                const u32x4_t c = sidx < 2 ? clo[i] : chi[i];
                const half8_t a = (sidx & 1) ? i8x8_to_half8(c.z, c.w, zbias[i]) : i8x8_to_half8(c.x, c.y, zbias[i]);
#pragma unroll
                for (int j = 0; j < kSJ; ++j)
                    if constexpr (!A8)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b[j][sidx], acc[i][j], 0, 0, 0);
            }
        }
      }
    };

    // prologue: tile 0 in flight
    if (0 < ktiles)
        issue(0, ring0, partial_t{});

    // this tile's per-channel scales, staged once in LDS for the epilogue;
    // the first barrier of the main loop publishes the LDS writes
#pragma unroll
    for (int c = tid; c < BN; c += C::kThreads)
        scale_lds[c] = n0 + c < n ? f16_bits_to_f32(scales[n0 + c]) : 0.0f;
    if constexpr (A8) {
#pragma unroll
        for (int r = tid; r < BM; r += C::kThreads)
            xscale_lds[r] = m0 + r < m ? f16_bits_to_f32(sx[m0 + r]) : 0.0f;
    }
    // Outliers are accumulated in code units (value / S, binary32), like the
    // dense products, so the epilogue's single multiply by S covers both.
    if constexpr (OL) {
        for (int e = tid; e < BN * kMfmaOutlierSlots; e += C::kThreads) {
            const int c = e / kMfmaOutlierSlots, slot = e % kMfmaOutlierSlots;
            int col = 0x7fffffff;
            float o = 0.0f;
            if (n0 + c < n && slot < ol.cap) {
                const int64_t at = (int64_t)(n0 + c) * ol.cap + slot;
                const int kk = ol.idx[at];
                if (kk >= 0 && kk < k) {
                    col = kk;
                    o = __fdiv_rn(ol.val[at], f16_bits_to_f32(scales[n0 + c]));
                }
            }
            ol_lds[e] = (int2v){col, __builtin_bit_cast(int, o)};
        }
    }
    // Step t (stage t % 2) waits for its own copies of tile t, the barrier
    // publishes everyone's copies and certifies that tile t-1's stage is no
    // longer read, tile t + 1 is copied into that stage while tile t is
    // multiplied.  FULL: tile t + 1 lies inside k (no per-chunk checks).
    //
    // A full step of a 256-channel fp16 tile spreads its copies over the
    // step: copy group g goes out right before MFMA group g (1-4% faster
    // than all copies at the top).  Other steps issue every copy at
    // the top.  Either way a scheduling barrier
    // pins the copies where they are: nothing ties them to the MFMAs, and
    // the scheduler would otherwise sink them below the whole step, right
    // before the wait for them.
    auto step = [&](int t, auto s, auto full) {
        constexpr int S = decltype(s)::value;
        constexpr bool kSpread = decltype(full)::value && kSpreadTile;
        QW_WAIT_VMCNT(0);
        ring_barrier();
        if constexpr (!kSpread) {
            if (decltype(full)::value || t + 1 < ktiles)
                issue(t + 1, ring(stage_t<1 - S>{}), full);
            __builtin_amdgcn_sched_barrier(0);
        }
        compute(ring(s), [&](int g) __attribute__((always_inline)) {
            if constexpr (kSpread) {
                issue_group(t + 1, ring(stage_t<1 - S>{}), g);
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    };
    // steady state: pairs of steps whose next tile is full
    int t = 0;
    for (; t + 2 < full_tiles; t += 2) {
        step(t, stage_t<0>{}, full_t{});
        step(t + 1, stage_t<1>{}, full_t{});
    }
    // at most three tiles remain: the last full pair's, and a ragged one
    for (int d = 0; d < 3; ++d) {
        if (t + d >= ktiles)
            break;
        if (d == 1)
            step(t + d, stage_t<1>{}, partial_t{});
        else
            step(t + d, stage_t<0>{}, partial_t{});
    }

    // ---- epilogue: scale, round to fp16, transpose through LDS, store ----
    // 32 x 32 output layout: accumulator r of lane l is row
    // 8 (r / 4) + 4 (l / 32) + (r % 4), column l % 32 of the MFMA tile, so
    // each group of 4 registers is 4 consecutive output channels of one
    // activation row.  They are scaled, rounded and written as 8 bytes into
    // the tile's [activation row][channel] image in LDS (row stride
    // 2 * BN + 16 bytes: the 32 rows one instruction touches fall on
    // distinct bank pairs); then the workgroup copies the image out in
    // 16-byte pieces, so every wave writes whole 512-byte row segments of Y
    // instead of scattered 8-byte pieces of 32 rows.
    ring_barrier(); // every wave is done reading the ring

    // OL: the side lists, one slot at a time.  The workgroup first gathers
    // G[c][r] = x[m0 + r][column of channel c's entry] for all of its
    // channels and activation rows into the free stage arrays (threads walk
    // the channels of one activation row, so a wave reads one row of X),
    // then every lane adds G * (value / S) to the accumulators it holds.
    // Unused entries have value 0 and gather a zero.
    if constexpr (OL) {
        constexpr int kGRow = BM + 2; // halves per channel row of G (padded: no bank conflicts)
        static_assert((BN / 2) * kGRow * 2 <= C::kStageAlloc, "G fits the stage arrays");
        auto gaddr = [&](int c, int r) -> _Float16 * {
            uint8_t *base = c < BN / 2 ? ring0 : ring1;
            return reinterpret_cast<_Float16 *>(base) + (c % (BN / 2)) * kGRow + r;
        };
        // Thread tid gathers channel tid % BN for rows tid / BN + i * kRStep.
        // The loads go out in batches of up to 32 (each a valid address:
        // entries without an outlier, and rows past m, load x[0][0] and keep
        // zero), so that their latencies overlap.
        static_assert(C::kThreads % BN == 0, "one channel per thread");
        constexpr int kRStep = C::kThreads / BN;
        constexpr int kPer = BM / kRStep;
        constexpr int kBatch = kPer < 32 ? kPer : 32;
        static_assert(kPer % kBatch == 0, "whole batches");
        const int gc = tid % BN, gr0 = tid / BN;
        const int slots = min(ol.cap, kMfmaOutlierSlots);
        for (int sl = 0; sl < slots; ++sl) {
            const int col = ol_lds[gc * kMfmaOutlierSlots + sl].x;
            const bool live = col != 0x7fffffff;
            for (int b0 = 0; b0 < kPer; b0 += kBatch) {
                uint16_t v[kBatch];
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int r = gr0 + (b0 + u) * kRStep;
                    const bool ok = live && m0 + r < m;
                    v[u] = x[ok ? (int64_t)(m0 + r) * k + col : 0];
                    v[u] = ok ? v[u] : (uint16_t)0;
                }
#pragma unroll
                for (int u = 0; u < kBatch; ++u)
                    *gaddr(gc, gr0 + (b0 + u) * kRStep) = __builtin_bit_cast(_Float16, v[u]);
            }
            ring_barrier();
#pragma unroll
            for (int i = 0; i < C::kSI; ++i) {
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const int c = wave * C::kWaveN + i * 32 + 8 * (rr / 4) + 4 * lgrp + rr % 4;
                    // (the component is copied out first: a bit cast applied to
                    // an ext-vector component in place reads component 0)
                    const int obits = ol_lds[c * kMfmaOutlierSlots + sl].y;
                    const float o = __builtin_bit_cast(float, obits);
#pragma unroll
                    for (int j = 0; j < kSJ; ++j)
                        acc[i][j][rr] += (float)*gaddr(c, j * 32 + lrow) * o;
                }
            }
            ring_barrier();
        }
    }

#pragma unroll
    for (int i = 0; i < C::kSI; ++i) {
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
            const int nl = wave * C::kWaveN + i * 32 + 8 * qd + 4 * lgrp;
            const float4v sc = *reinterpret_cast<const float4v *>(scale_lds + nl);
#pragma unroll
            for (int j = 0; j < kSJ; ++j) {
                // rows [0, BM/2) of the image live in stage 0's array
                uint8_t *img = j < kSJ / 2 ? ring0 + (j * 32 + lrow) * C::kYRow
                                           : ring1 + (j * 32 - BM / 2 + lrow) * C::kYRow;
                // W8A16: acc * S[n].  W8A8: float(acc) * (S[n] * Sx[m]); the
                // product of two fp16 scales is exact in fp32.
                auto val = [&](int e) -> float {
                    if constexpr (A8)
                        return (float)acc[i][j][4 * qd + e] * (sc[e] * xscale_lds[j * 32 + lrow]);
                    else
                        return acc[i][j][4 * qd + e] * sc[e];
                };
                const uint32_t o0 = f32_to_f16_bits(val(0));
                const uint32_t o1 = f32_to_f16_bits(val(1));
                const uint32_t o2 = f32_to_f16_bits(val(2));
                const uint32_t o3 = f32_to_f16_bits(val(3));
                *reinterpret_cast<u32x2_t *>(img + nl * 2) = (u32x2_t){o0 | (o1 << 16), o2 | (o3 << 16)};
            }
        }
    }
    ring_barrier();
    constexpr int kRowChunks = BN / 8; // 16-byte pieces per output row
    const bool vec_ok = (n % 8) == 0 && n0 + BN <= n;
    const int rows = min(BM, m - m0);
    for (int c = tid; c < rows * kRowChunks; c += C::kThreads) {
        const int row = c / kRowChunks;
        const int cc = c % kRowChunks;
        const uint8_t *img = row < BM / 2 ? ring0 + row * C::kYRow : ring1 + (row - BM / 2) * C::kYRow;
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(img + cc * 16);
        uint16_t *dst = y + (int64_t)(m0 + row) * n + n0 + cc * 8;
        if (vec_ok) {
            // streamed past the caches: Y is not read again here, and dirty
            // lines left in L2 would be written back at the end of the kernel
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(dst));
        } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n0 + cc * 8 + e < n)
                    dst[e] = (uint16_t)(w[e / 2] >> (16 * (e % 2)));
        }
    }
}

// ---------------------------------------------------------------------------
// Ping-pong variant for grids of 256 x 256 tiles: 8 waves per workgroup,
// two per SIMD, in two groups of four (one wave per SIMD each).  Group 0
// computes activation rows [0, 128) of the tile, group 1 rows [128, 256);
// wave w % 4 of either group owns output channels [64 (w % 4), +64), so a
// wave's share of a k step is the same 64 x 128 block (8 MFMA tiles of
// 32 x 32, 32 MFMAs) as in the 4-wave kernel above.
//
// The two groups run half a k step apart, separated by workgroup barriers:
// while one group's waves issue their MFMAs back to back (registers only),
// the other group's waves read their operands of the next k step from LDS
// and issue their share of the copies of a later tile.  Each SIMD thus
// holds one wave in an MFMA run and one wave in a memory phase at any time,
// instead of two waves that contend for the same units.  Phases (p):
//
//   group 0: p = 2t     read tile t from LDS, copy tile t + 2 (its half)
//            p = 2t + 1 MFMAs of tile t
//   group 1: p = 2t + 1 read tile t from LDS, copy tile t + 2 (its half)
//            p = 2t + 2 MFMAs of tile t
//
// Every wave executes the same number of barriers: 2T over the k loop of
// T tiles, then three in the epilogue.  Three LDS stages (48 KiB each) hold
// tiles t, t + 1 and t + 2: the stage tile t + 2 goes into held tile t - 1,
// which group 1 read in phase 2t - 1, before the barrier that opens phase
// 2t.  A wave's copies of tile u are waited for at the end of phase 2u - 1
// (its own wait counter, then the barrier): they were issued in phase
// 2u - 4 or 2u - 3, so their latency hides behind two to three phases.
// ---------------------------------------------------------------------------
namespace pp {
constexpr int kBN = 256;                          // output channels per workgroup
constexpr int kBM = 256;                          // activation rows per workgroup
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;
constexpr int kSI = 2;                            // 32-channel MFMA tiles per wave
constexpr int kSJ = 4;                            // 32-row MFMA tiles per wave
constexpr int kGroupRows = kSJ * 32;              // activation rows per group
constexpr int kWBytes = kBN * kBK;                // int8 weight tile per stage
// epilogue image of one group's rows, [128][256] fp16 with rows padded by
// 16 bytes; rows [0, 64) in stage 0's array, [64, 128) in stage 1's
constexpr int kYRow = kBN * 2 + 16;
static_assert(4 * kSI * 32 == kBN && 2 * kGroupRows == kBM, "wave layout");

// A8: int8 activation codes (W8A8), laid out in LDS like the weight rows
// (16 rows per 1 KiB copy); otherwise fp16 (8 rows per copy).
template <bool A8>
struct Cfg {
    static constexpr int kXBytes = kBM * kBK * (A8 ? 1 : 2); // activation tile per stage
    static constexpr int kStage = kWBytes + kXBytes;
    static constexpr int kWInstr = kWBytes / 1024 / kWaves;  // copies per wave per tile
    static constexpr int kXInstr = kXBytes / 1024 / kWaves;
    static constexpr int kCopies = kWInstr + kXInstr;
    // a stage array also holds half a group's epilogue image
    static constexpr int kImageHalf = (kGroupRows / 2) * kYRow;
    static constexpr int kStageAlloc = kStage > kImageHalf ? kStage : kImageHalf;
    static_assert(kWInstr * 1024 * kWaves == kWBytes && kXInstr * 1024 * kWaves == kXBytes, "copy split");
    static_assert(A8 || kXInstr % 2 == 0, "fp16 activation copies alternate between the two 8-row swizzle phases");
};
} // namespace pp

static_assert(pp::kBM * kPingPongMaxK * 2 <= (int64_t(1) << 31), "buffer range");

// A8 (W8A8): xv holds int8 activation codes with one fp16 scale per row in
// sx; the MFMA is v_mfma_i32_32x32x32_i8 (two per 64-wide k step and tile,
// no casts), int32 accumulators, and the epilogue multiplies by S[n] * Sx[m].
// Otherwise xv is fp16 and sx unused.
template <bool A8, bool OL, bool ZP>
__global__ __launch_bounds__(pp::kThreads) void mfma_pp_kernel(
    const void *__restrict__ xv, const uint16_t *__restrict__ sx, const int8_t *__restrict__ q,
    const uint16_t *__restrict__ scales, const int8_t *__restrict__ zeros, OutlierList ol,
    uint16_t *__restrict__ y, int m, int n, int k, int tiles_m, int tiles_n, int group)
{
    using namespace pp;
    using C = Cfg<A8>;
    constexpr int kStage = C::kStage;
    constexpr int kWInstr = C::kWInstr;
    constexpr int kXInstr = C::kXInstr;
    constexpr int kCopies = C::kCopies;
    static_assert(!A8 || (!OL && !ZP), "W8A8 takes symmetric codes without side lists");
    const uint16_t *__restrict__ x = static_cast<const uint16_t *>(xv);
    __shared__ __attribute__((aligned(1024))) uint8_t ring0[C::kStageAlloc];
    __shared__ __attribute__((aligned(1024))) uint8_t ring1[C::kStageAlloc];
    __shared__ __attribute__((aligned(1024))) uint8_t ring2[C::kStageAlloc];
    __shared__ __attribute__((aligned(16))) float scale_lds[kBN];
    __shared__ __attribute__((aligned(16))) float xscale_lds[A8 ? kBM : 1];
    // OL: the workgroup's side lists, (column, value / S as float bits) per
    // slot; unused slots hold column INT_MAX
    __shared__ __attribute__((aligned(16))) int2v ol_lds[OL ? kBN * kMfmaOutlierSlots : 1];
    auto ring = [&](auto s) -> uint8_t * {
        if constexpr (decltype(s)::value == 0)
            return ring0;
        else if constexpr (decltype(s)::value == 1)
            return ring1;
        else
            return ring2;
    };

    const int tid = threadIdx.x;
    const int lane = __lane_id();
    const int wave = __builtin_amdgcn_readlane(tid / kWave, 0);
    const int grp = wave / 4;
    const int nw = wave % 4;

    const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
    const int gsize = group * tiles_m;
    const int gi = tile / gsize;
    const int gl = tile - gi * gsize;
    const int gw = min(group, tiles_n - gi * group);
    const int tn = gi * group + gl % gw;
    const int tm = gl / gw;
    const int n0 = tn * kBN;
    const int m0 = tm * kBM;
    const int ktiles = (k + kBK - 1) / kBK;
    const int full_tiles = (k % kBK) != 0 ? ktiles - 1 : ktiles;

    // Copy sources: as in the 4-wave kernel, with 8 waves sharing a tile.
    // Copy i of a wave covers rows 16 i (weight) or 8 i (activations) below
    // its copy 0, so one lane offset per swizzle phase serves all copies and
    // the rest goes into the scalar offset.  Rows past n or m are not
    // clamped: they lie past the end of the buffer range, and such reads
    // return zeros (only outputs that are never stored depend on them).
    const int wchunk = (lane % 4) ^ wslot(lane / 4);
    const int xchunk_even = (lane % 8) ^ xslot(lane / 8);
    const int xchunk_odd = (lane % 8) ^ xslot(8 + lane / 8);
    constexpr int kXE = A8 ? 1 : 2; // bytes per activation element
    const uint32_t woff = (uint32_t)((wave * kWInstr * 16 + lane / 4) * k + wchunk * 16);
    // A8: activation copy i covers rows 16 i below copy 0, like the weight
    const uint32_t xrow0 = (uint32_t)(A8 ? wave * kXInstr * 16 + lane / 4 : wave * kXInstr * 8 + lane / 8);
    const uint32_t xoff_even = A8 ? xrow0 * k + wchunk * 16 : (xrow0 * k + xchunk_even * 8) * 2;
    const uint32_t xoff_odd = A8 ? xoff_even : ((xrow0 + 8) * k + xchunk_odd * 8) * 2;
    // (the scalar offset of activation copy i, written out at each use: as a
    // lambda or a template helper it kept the host pass from emitting the
    // kernels' launch stubs)
    const int8_t *wtile = q + (int64_t)n0 * k;
    const uint8_t *xtile = static_cast<const uint8_t *>(xv) + (int64_t)m0 * k * kXE;
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t *>(wtile), (short)0,
        static_cast<int>(static_cast<uint32_t>(min((int64_t)kBN, (int64_t)(n - n0)) * k)), kBufferFlags);
    const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(xtile), (short)0,
        static_cast<int>(static_cast<uint32_t>(min((int64_t)kBM, (int64_t)(m - m0)) * k * kXE)), kBufferFlags);

    // this wave's share of the copies of tile kt into stage array st
    auto issue_full = [&](int kt, uint8_t *st) {
        const int k0 = kt * kBK;
#pragma unroll
        for (int i = 0; i < kWInstr; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wrsrc, (lds_ptr_t)(st + (wave * kWInstr + i) * 1024), 16,
                                                     (int)woff, k0 + i * 16 * k, 0, 0);
#pragma unroll
        for (int i = 0; i < kXInstr; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xrsrc, (lds_ptr_t)(st + kWBytes + (wave * kXInstr + i) * 1024), 16,
                (int)((i & 1) ? xoff_odd : xoff_even), (A8 ? k0 + i * 16 * k : (k0 + (i & ~1) * 8 * k) * 2), 0, 0);
    };
    // The ragged last tile: activation chunks past k are zero-filled, so
    // whatever the weight chunks past k hold (codes of the next row, or
    // zeros past the buffer range) multiplies zeros.
    auto issue_partial = [&](int kt, uint8_t *st) {
        const int k0 = kt * kBK;
#pragma unroll
        for (int i = 0; i < kWInstr; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wrsrc, (lds_ptr_t)(st + (wave * kWInstr + i) * 1024), 16,
                                                     (int)woff, k0 + i * 16 * k, 0, 0);
#pragma unroll
        for (int i = 0; i < kXInstr; ++i) {
            uint8_t *dst = st + kWBytes + (wave * kXInstr + i) * 1024;
            const int gk = k0 + (A8 ? wchunk * 16 : ((i & 1) ? xchunk_odd : xchunk_even) * 8);
            if (gk < k)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xrsrc, (lds_ptr_t)dst, 16,
                                                         (int)((i & 1) ? xoff_odd : xoff_even), (A8 ? k0 + i * 16 * k : (k0 + (i & ~1) * 8 * k) * 2), 0, 0);
            else
                *reinterpret_cast<u32x4_t *>(dst + lane * 16) = (u32x4_t){0u, 0u, 0u, 0u};
        }
    };
    // FULL: tile kt is known to lie inside k
    auto issue = [&](int kt, uint8_t *st, auto full) {
        if constexpr (decltype(full)::value) {
            issue_full(kt, st);
        } else {
            if (kt < full_tiles)
                issue_full(kt, st);
            else if (kt < ktiles)
                issue_partial(kt, st);
        }
    };
    // End of phase 2u - 1: this wave's copies of tile u are done; the batch
    // of tile u + 1 it issued since may stay in flight (FULL: that batch was
    // a full tile).  Written as inline asm behind a scheduling barrier: the
    // builtin form alone was moved past the phase's barrier, and either form
    // ahead of the MFMAs.  The builtin beside it tells the compiler's own
    // wait-count bookkeeping what has completed.
    auto wait_tile = [&](int u, auto full) {
        static_assert(kCopies == 6 || kCopies == 4, "the wait below names the batch size");
        __builtin_amdgcn_sched_barrier(0);
        if (decltype(full)::value || u + 1 < full_tiles) {
            if constexpr (kCopies == 6)
                __asm__ __volatile__("s_waitcnt vmcnt(6)" ::: "memory");
            else
                __asm__ __volatile__("s_waitcnt vmcnt(4)" ::: "memory");
            QW_WAIT_VMCNT(kCopies);
        } else {
            __asm__ __volatile__("s_waitcnt vmcnt(0)" ::: "memory");
            QW_WAIT_VMCNT(0);
        }
    };
    // A phase boundary.  The scheduling barriers keep the compiler from
    // moving any instruction (the MFMAs above all, which touch no memory)
    // across the workgroup barrier into the neighbouring phase.
    auto phase_end = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        ring_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    // operand layout of v_mfma_f32_32x32x16_f16 as in the 4-wave kernel
    const int lrow = lane % 32;
    const int lgrp = lane / 32;
    // The row bases have bits 4..7 clear, so the swizzled 16-byte chunk
    // c ^ slot of chunk c = c0 + s is the base's chunk c0 XOR s: one lane
    // offset per operand, the others one XOR away (kept out of registers
    // across the loop).
    const int wrow = nw * (kSI * 32) + lrow; // + 32 i
    const int w_off0 = wrow * kBK + 16 * ((2 * lgrp) ^ wslot(wrow));
    const int xrow = grp * kGroupRows + lrow; // + 32 j
    // A8: the activation rows are read like the weight rows (chunks 2g, 2g+1)
    const int x_off0 = A8 ? kWBytes + xrow * kBK + 16 * ((2 * lgrp) ^ wslot(xrow))
                          : kWBytes + xrow * 2 * kBK + 16 * ((4 * lgrp) ^ xslot(xrow));

    using acc_t = std::conditional_t<A8, int16v, float16v>;
    acc_t acc[kSI][kSJ];
#pragma unroll
    for (int i = 0; i < kSI; ++i)
#pragma unroll
        for (int j = 0; j < kSJ; ++j)
            acc[i][j] = (acc_t){};
    half2_t zbias[kSI];
#pragma unroll
    for (int i = 0; i < kSI; ++i) {
        const int zr = n0 + wrow + 32 * i;
        zbias[i] = zero_point_bias(ZP && zr < n ? (int)zeros[zr] : 0);
    }

    // Operands of one k step: the weight codes are cast to fp16 in the
    // memory phase, right after their LDS reads, so that the MFMA phase is
    // MFMAs only (cast between the MFMAs, the casts' VALU work did not
    // overlap them and stretched the MFMA phase by about 40%).
    half8_t a[kSI][4];
    half8_t b[kSJ][4];
    // A8: the 16 codes of chunk 2g + s per lane, weight (A) and activation
    // (B) operands of v_mfma_i32_32x32x32_i8 alike, as in the 4-wave kernel
    u32x4_t a8[kSI][2], b8[kSJ][2];
    auto load = [&](const uint8_t *st) {
        if constexpr (A8) {
            int w_off1, x_off1;
            __asm__ __volatile__("v_xor_b32 %0, 16, %1" : "=v"(w_off1) : "v"(w_off0));
            __asm__ __volatile__("v_xor_b32 %0, 16, %1" : "=v"(x_off1) : "v"(x_off0));
#pragma unroll
            for (int i = 0; i < kSI; ++i) {
                a8[i][0] = *reinterpret_cast<const u32x4_t *>(st + w_off0 + i * 32 * kBK);
                a8[i][1] = *reinterpret_cast<const u32x4_t *>(st + w_off1 + i * 32 * kBK);
            }
#pragma unroll
            for (int j = 0; j < kSJ; ++j) {
                b8[j][0] = *reinterpret_cast<const u32x4_t *>(st + x_off0 + j * 32 * kBK);
                b8[j][1] = *reinterpret_cast<const u32x4_t *>(st + x_off1 + j * 32 * kBK);
            }
            return;
        }
        int w_off1, x_off[4];
        x_off[0] = x_off0;
        // (volatile: computed here, in the memory phase, rather than hoisted
        // out of the loop into registers held across it)
        __asm__ __volatile__("v_xor_b32 %0, 16, %1" : "=v"(w_off1) : "v"(w_off0));
        __asm__ __volatile__("v_xor_b32 %0, 16, %1" : "=v"(x_off[1]) : "v"(x_off0));
        __asm__ __volatile__("v_xor_b32 %0, 32, %1" : "=v"(x_off[2]) : "v"(x_off0));
        __asm__ __volatile__("v_xor_b32 %0, 48, %1" : "=v"(x_off[3]) : "v"(x_off0));
        u32x4_t clo[kSI], chi[kSI];
#pragma unroll
        for (int i = 0; i < kSI; ++i) {
            clo[i] = *reinterpret_cast<const u32x4_t *>(st + w_off0 + i * 32 * kBK);
            chi[i] = *reinterpret_cast<const u32x4_t *>(st + w_off1 + i * 32 * kBK);
        }
#pragma unroll
        for (int sidx = 0; sidx < 4; ++sidx)
#pragma unroll
            for (int j = 0; j < kSJ; ++j)
                b[j][sidx] = *reinterpret_cast<const half8_t *>(st + x_off[sidx] + j * 32 * 2 * kBK);
#pragma unroll
        for (int i = 0; i < kSI; ++i) {
            a[i][0] = i8x8_to_half8(clo[i].x, clo[i].y, zbias[i]);
            a[i][1] = i8x8_to_half8(clo[i].z, clo[i].w, zbias[i]);
            a[i][2] = i8x8_to_half8(chi[i].x, chi[i].y, zbias[i]);
            a[i][3] = i8x8_to_half8(chi[i].z, chi[i].w, zbias[i]);
        }
    };
    auto compute = [&]() {
        if constexpr (A8) {
#pragma unroll
            for (int sidx = 0; sidx < 2; ++sidx)
#pragma unroll
                for (int i = 0; i < kSI; ++i)
#pragma unroll
                    for (int j = 0; j < kSJ; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(int4v, a8[i][sidx]),
                                                                         __builtin_bit_cast(int4v, b8[j][sidx]),
                                                                         acc[i][j], 0, 0, 0);
        } else {
#pragma unroll
            for (int sidx = 0; sidx < 4; ++sidx)
#pragma unroll
                for (int i = 0; i < kSI; ++i)
#pragma unroll
                    for (int j = 0; j < kSJ; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i][sidx], b[j][sidx], acc[i][j], 0, 0, 0);
        }
    };
    // memory phase of tile t (stage S): copies of tile t + 2, then operands
    auto mem = [&](int t, auto s, auto full) {
        constexpr int S = decltype(s)::value;
        issue(t + 2, ring(stage_t<(S + 2) % 3>{}), full);
        __builtin_amdgcn_sched_barrier(0);
        load(ring(s));
    };
    using full_t = std::integral_constant<bool, true>;
    using partial_t = std::integral_constant<bool, false>;

    // prologue: tiles 0 and 1 in flight, scales staged, tile 0 landed
    issue(0, ring0, partial_t{});
    issue(1, ring1, partial_t{});
    for (int c = tid; c < kBN; c += kThreads)
        scale_lds[c] = n0 + c < n ? f16_bits_to_f32(scales[n0 + c]) : 0.0f;
    if constexpr (A8) {
        for (int r = tid; r < kBM; r += kThreads)
            xscale_lds[r] = m0 + r < m ? f16_bits_to_f32(sx[m0 + r]) : 0.0f;
    }
    if constexpr (OL) {
        for (int e = tid; e < kBN * kMfmaOutlierSlots; e += kThreads) {
            const int c = e / kMfmaOutlierSlots, slot = e % kMfmaOutlierSlots;
            int col = 0x7fffffff;
            float o = 0.0f;
            if (n0 + c < n && slot < ol.cap) {
                const int64_t at = (int64_t)(n0 + c) * ol.cap + slot;
                const int kk = ol.idx[at];
                if (kk >= 0 && kk < k) {
                    col = kk;
                    o = __fdiv_rn(ol.val[at], f16_bits_to_f32(scales[n0 + c]));
                }
            }
            ol_lds[e] = (int2v){col, __builtin_bit_cast(int, o)};
        }
    }
    wait_tile(0, partial_t{});
    phase_end();

    // The steady loop runs while tiles t + 2 ... t + 4, copied by its three
    // steps, lie inside k; at most five steps remain after it.
    auto run = [&](auto &&body) {
        int t = 0;
        for (; t + 5 <= full_tiles; t += 3) {
            body(t, stage_t<0>{}, full_t{});
            body(t + 1, stage_t<1>{}, full_t{});
            body(t + 2, stage_t<2>{}, full_t{});
        }
        static_for<0, 5>([&](auto d) {
            if (t + d < ktiles)
                body(t + d, stage_t<decltype(d)::value % 3>{}, partial_t{});
        });
    };
    if (grp == 0) {
        run([&](int t, auto s, auto full) {
            mem(t, s, full);
            phase_end(); // end of phase 2t
            compute();
            wait_tile(t + 1, full);
            phase_end(); // end of phase 2t + 1
        });
    } else {
        phase_end(); // end of phase 0
        run([&](int t, auto s, auto full) {
            mem(t, s, full);
            wait_tile(t + 1, full);
            phase_end(); // end of phase 2t + 1
            compute();
            if (t + 1 < ktiles)
                phase_end(); // end of phase 2t + 2
        });
    }

    // ---- epilogue: one group at a time through an LDS image of its rows ----
    // group 0 writes its image in phase 2T (all stages are free: group 1
    // read the last tile in phase 2T - 1) while group 1 finishes its MFMAs
    auto write_image = [&]() {
#pragma unroll
        for (int i = 0; i < kSI; ++i) {
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int nl = nw * (kSI * 32) + i * 32 + 8 * qd + 4 * lgrp;
                const float4v sc = *reinterpret_cast<const float4v *>(scale_lds + nl);
#pragma unroll
                for (int j = 0; j < kSJ; ++j) {
                    uint8_t *img = j < kSJ / 2 ? ring0 + (j * 32 + lrow) * kYRow
                                               : ring1 + (j * 32 - kGroupRows / 2 + lrow) * kYRow;
                    // W8A16: acc * S[n].  W8A8: float(acc) * (S[n] * Sx[m]);
                    // the product of two fp16 scales is exact in fp32.
                    auto val = [&](int e) -> float {
                        if constexpr (A8)
                            return (float)acc[i][j][4 * qd + e] *
                                   (sc[e] * xscale_lds[grp * kGroupRows + j * 32 + lrow]);
                        else
                            return acc[i][j][4 * qd + e] * sc[e];
                    };
                    const uint32_t o0 = f32_to_f16_bits(val(0));
                    const uint32_t o1 = f32_to_f16_bits(val(1));
                    const uint32_t o2 = f32_to_f16_bits(val(2));
                    const uint32_t o3 = f32_to_f16_bits(val(3));
                    *reinterpret_cast<u32x2_t *>(img + nl * 2) = (u32x2_t){o0 | (o1 << 16), o2 | (o3 << 16)};
                }
            }
        }
    };
    constexpr int kRowChunks = kBN / 8;
    const bool vec_ok = (n % 8) == 0 && n0 + kBN <= n;
    auto store_rows = [&](int g) {
        const int r0 = m0 + g * kGroupRows;
        const int rows = min(kGroupRows, m - r0);
        for (int c = tid; c < rows * kRowChunks; c += kThreads) {
            const int row = c / kRowChunks;
            const int cc = c % kRowChunks;
            const uint8_t *img = row < kGroupRows / 2 ? ring0 + row * kYRow : ring1 + (row - kGroupRows / 2) * kYRow;
            const u32x4_t v = *reinterpret_cast<const u32x4_t *>(img + cc * 16);
            uint16_t *dst = y + (int64_t)(r0 + row) * n + n0 + cc * 8;
            if (vec_ok) {
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(dst));
            } else {
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (n0 + cc * 8 + e < n)
                        dst[e] = (uint16_t)(w[e / 2] >> (16 * (e % 2)));
            }
        }
    };
    if constexpr (OL) {
        // Outlier side lists, one slot at a time, after both groups' MFMAs
        // (end of phase 2T): the workgroup gathers G[c][r] = x[m0 + r][column
        // of channel c's entry] for all 256 channels and rows into the three
        // stage arrays (86 channels each, rows padded by 2 halves), then every
        // lane adds G * (value / S) to the accumulators it holds.  Unused
        // entries have value 0 and gather a zero.
        ring_barrier();
        constexpr int kGRow = kBM + 2;
        constexpr int kGPer = 86;
        static_assert(kGPer * kGRow * 2 <= kStage && 3 * kGPer >= kBN, "G fits the stage arrays");
        auto gaddr = [&](int c, int r) -> _Float16 * {
            const int a = c / kGPer;
            uint8_t *base = a == 0 ? ring0 : (a == 1 ? ring1 : ring2);
            return reinterpret_cast<_Float16 *>(base) + (c - a * kGPer) * kGRow + r;
        };
        constexpr int kRStep = kThreads / kBN;
        constexpr int kPer = kBM / kRStep;
        constexpr int kBatch = 32;
        static_assert(kThreads % kBN == 0 && kPer % kBatch == 0, "gather split");
        const int gc = tid % kBN, gr0 = tid / kBN;
        const int slots = min(ol.cap, kMfmaOutlierSlots);
        for (int sl = 0; sl < slots; ++sl) {
            const int col = ol_lds[gc * kMfmaOutlierSlots + sl].x;
            const bool live = col != 0x7fffffff;
            for (int b0 = 0; b0 < kPer; b0 += kBatch) {
                uint16_t v[kBatch];
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int r = gr0 + (b0 + u) * kRStep;
                    const bool ok = live && m0 + r < m;
                    v[u] = x[ok ? (int64_t)(m0 + r) * k + col : 0];
                    v[u] = ok ? v[u] : (uint16_t)0;
                }
#pragma unroll
                for (int u = 0; u < kBatch; ++u)
                    *gaddr(gc, gr0 + (b0 + u) * kRStep) = __builtin_bit_cast(_Float16, v[u]);
            }
            ring_barrier();
#pragma unroll
            for (int i = 0; i < kSI; ++i) {
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const int c = nw * (kSI * 32) + i * 32 + 8 * (rr / 4) + 4 * lgrp + rr % 4;
                    // (copied out first: a bit cast of an ext-vector
                    // component in place reads component 0)
                    const int obits = ol_lds[c * kMfmaOutlierSlots + sl].y;
                    const float o = __builtin_bit_cast(float, obits);
#pragma unroll
                    for (int j = 0; j < kSJ; ++j)
                        acc[i][j][rr] += (float)*gaddr(c, grp * kGroupRows + j * 32 + lrow) * o;
                }
            }
            ring_barrier();
        }
    }
    if (grp == 0)
        write_image();
    ring_barrier();
    store_rows(0);
    ring_barrier();
    if (grp == 1)
        write_image();
    ring_barrier();
    store_rows(1);
}

template <int BN, int BM, bool A8>
int64_t slots_per_cu();

// Weight-tile columns per group of the tile order.  An XCD holds about r =
// min(its share of the grid, its resident workgroups) tiles at once; as an
// a x (r / a) block of weight x activation tiles they fetch a * BN weight
// rows and (r / a) * BM activation rows per k step, least at
// a = sqrt(r * BM * e / BN) with e the bytes of one activation element.
// With few activation tiles (prefill: 4) the block needs at least
// r / tiles_m columns; a group that wide also makes consecutive workgroups
// share an activation tile, which measured 3-7% faster there than narrower
// groups.  Measured on MI355X against one column per group: 5-14% faster
// for the W8A8 tiles and 1-7% for the fp16 tiles with 256 weight rows; the
// fp16 tiles with 128 weight rows ran 1-5% slower grouped, at either width,
// and keep one.
template <int BN, int BM, bool A8>
int group_width(int64_t blocks, int64_t tiles_m, int64_t tiles_n)
{
    if constexpr (!A8 && BN == 128)
        return 1;
    const int64_t share = (blocks + 7) / 8;
    const int64_t resident = slots_per_cu<BN, BM, A8>() * (int64_t)device_cu_count() / 8;
    const double r = (double)std::max<int64_t>(1, std::min(share, resident));
    int64_t a = std::llround(std::sqrt(r * BM * (A8 ? 1 : 2) / BN));
    a = std::max<int64_t>(a, ((int64_t)r + tiles_m - 1) / tiles_m);
    return (int)std::max<int64_t>(1, std::min(a, tiles_n));
}

template <int NW, int BN, int BM, bool A8>
hipError_t launch_dma(const void *x, const uint16_t *sx, const int8_t *q, const uint16_t *scales,
                      const int8_t *zeros, OutlierList ol, uint16_t *y, int64_t m, int64_t n, int64_t k,
                      hipStream_t stream)
{
    const int64_t tiles_m = (m + BM - 1) / BM;
    const int64_t tiles_n = (n + BN - 1) / BN;
    const int64_t blocks = tiles_m * tiles_n;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    const int group = group_width<BN, BM, A8>(blocks, tiles_m, tiles_n);
    if constexpr (!A8) {
        if (ol.idx != nullptr) {
            if (ol.cap > kMfmaOutlierSlots)
                return hipErrorInvalidValue;
            hipLaunchKernelGGL((mfma_gemm_dma_kernel<NW, BN, BM, false, true>), dim3((unsigned)blocks),
                               dim3(NW * kWave), 0, stream, x, sx, q, scales, zeros, ol, y, (int)m, (int)n,
                               (int)k, (int)tiles_m, (int)tiles_n, group);
            return hipGetLastError();
        }
    }
    if (ol.idx != nullptr)
        return hipErrorInvalidValue;
    if constexpr (!A8) {
        if (zeros != nullptr) {
            hipLaunchKernelGGL((mfma_gemm_dma_kernel<NW, BN, BM, false, false, true>), dim3((unsigned)blocks),
                               dim3(NW * kWave), 0, stream, x, sx, q, scales, zeros, ol, y, (int)m, (int)n,
                               (int)k, (int)tiles_m, (int)tiles_n, group);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((mfma_gemm_dma_kernel<NW, BN, BM, A8>), dim3((unsigned)blocks), dim3(NW * kWave),
                       0, stream, x, sx, q, scales, zeros, ol, y, (int)m, (int)n, (int)k, (int)tiles_m,
                       (int)tiles_n, group);
    return hipGetLastError();
}

// Workgroups of this tile shape one CU holds at once (registers and LDS),
// queried once per device.  Host threads may race on the first query; they
// store the same value.
template <int BN, int BM, bool A8>
int64_t slots_per_cu()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 1;
    int blocks = cached[dev].load(std::memory_order_relaxed);
    if (blocks == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, mfma_gemm_dma_kernel<4, BN, BM, A8>,
                                                        4 * kWave, 0) != hipSuccess || blocks < 1)
            blocks = 1;
        cached[dev].store(blocks, std::memory_order_relaxed);
    }
    return blocks;
}

template <int BN, int BM, bool A8>
bool fills(int64_t m, int64_t n)
{
    const int64_t tiles = ((n + BN - 1) / BN) * ((m + BM - 1) / BM);
    // The fp16 128 x 128 tile is counted at two workgroups per CU even where
    // its registers allow three: per-shape tuning measured it fastest at 256
    // rows (N = 27392), where counting the third slot would pass it over
    // for 128 x 64.
    int64_t per_cu = slots_per_cu<BN, BM, A8>();
    if (!A8 && BN == 128 && BM == 128 && per_cu > 2)
        per_cu = 2;
    const int64_t slots = per_cu * (int64_t)device_cu_count();
    return 4 * tiles >= 3 * slots;
}

// The ping-pong tile (fp16 activations) where its grid covers at least half
// the CUs (one workgroup per CU) and rounding m up to 256 rows costs at most
// 10% more rows than rounding it to 64 (the smallest 4-wave tile).
// Measured on MI355X against the 4-wave tiles: 10-13% faster at 512 x 4096
// x 27392, 8% at 2048 x 4096 x 4608 (144 tiles), even at 4096 x 1024 x
// 4096; 20% slower at 256 x 4096 x 27392 (107 tiles).
bool pp_fills(int64_t m, int64_t n, int64_t k)
{
    if (k > kPingPongMaxK)
        return false;
    const int64_t tiles = ((m + pp::kBM - 1) / pp::kBM) * ((n + pp::kBN - 1) / pp::kBN);
    const int64_t rows256 = (m + 255) / 256 * 256, rows64 = (m + 63) / 64 * 64;
    return 2 * tiles >= (int64_t)device_cu_count() && 10 * rows256 <= 11 * rows64;
}

// PP: the ping-pong tile may be chosen.  Calls with outlier side lists keep
// the 4-wave tiles: the ping-pong kernel's epilogue gather of the side
// lists' activation columns, one workgroup per CU with nothing to overlap
// it, measured 54% above the plain GEMM on 4096 x 1024 x 4096 (one slot)
// against 43% for the 256 x 128 tile.
template <bool A8>
int tile_choice(int64_t m, int64_t n, int64_t k, bool pp = true)
{
    if (pp && pp_fills(m, n, k))
        return 256256;
    // largest tile first (more reuse per byte staged); 256 x 64 before
    // 128 x 128 (same area, half the activation bytes per tile)
    if (fills<256, 128, A8>(m, n))
        return 256128;
    if (fills<256, 64, A8>(m, n))
        return 256064;
    // W8A8: the 128 x 128 tile holds four workgroups per CU (int8 activation
    // tiles are half the LDS), so it fills the chip only where 256 x 64
    // already does and is never the choice
    if (!A8 && fills<128, 128, A8>(m, n))
        return 128128;
    return 128064;
}

// Ping-pong launch: one 512-thread workgroup per 256 x 256 tile, one per CU
// (144 KiB of LDS).  Grouped tile order as for the 4-wave tiles, with one
// resident workgroup per CU.
template <bool A8>
hipError_t launch_pp(const void *x, const uint16_t *sx, const int8_t *q, const uint16_t *scales,
                     const int8_t *zeros, OutlierList ol, uint16_t *y, int64_t m, int64_t n, int64_t k,
                     hipStream_t stream)
{
    const int64_t tiles_m = (m + pp::kBM - 1) / pp::kBM;
    const int64_t tiles_n = (n + pp::kBN - 1) / pp::kBN;
    const int64_t blocks = tiles_m * tiles_n;
    if (blocks > 0x7fffffff || k < 1 || k > kPingPongMaxK || (ol.idx != nullptr && ol.cap > kMfmaOutlierSlots))
        return hipErrorInvalidValue;
    const int64_t share = (blocks + 7) / 8;
    const int64_t resident = std::max<int64_t>(1, (int64_t)device_cu_count() / 8);
    const double r = (double)std::max<int64_t>(1, std::min(share, resident));
    int64_t a = std::llround(std::sqrt(r * pp::kBM * (A8 ? 1 : 2) / pp::kBN));
    a = std::max<int64_t>(a, ((int64_t)r + tiles_m - 1) / tiles_m);
    const int group = (int)std::max<int64_t>(1, std::min(a, tiles_n));
#define QW_PP_LAUNCH(A, O, Z)                                                                                   \
    hipLaunchKernelGGL((mfma_pp_kernel<A, O, Z>), dim3((unsigned)blocks), dim3(pp::kThreads), 0, stream, x, sx, q,  \
                       scales, zeros, ol, y, (int)m, (int)n, (int)k, (int)tiles_m, (int)tiles_n, group)
    if constexpr (A8) {
        if (ol.idx != nullptr || zeros != nullptr)
            return hipErrorInvalidValue;
        QW_PP_LAUNCH(true, false, false);
    } else {
        // side lists come with symmetric codes only (as in the 4-wave kernels)
        if (ol.idx != nullptr)
            QW_PP_LAUNCH(false, true, false);
        else if (zeros != nullptr)
            QW_PP_LAUNCH(false, false, true);
        else
            QW_PP_LAUNCH(false, false, false);
    }
#undef QW_PP_LAUNCH
    return hipGetLastError();
}

template <bool A8>
hipError_t launch_tiles(const void *x, const uint16_t *sx, const int8_t *q, const uint16_t *scales,
                        const int8_t *zeros, OutlierList ol, uint16_t *y, int64_t m, int64_t n, int64_t k,
                        hipStream_t stream, int forced_tile = 0)
{
    if (k > kMfmaMaxK) // the entry points route such rows elsewhere
        return hipErrorInvalidValue;
    const int tile = forced_tile != 0 ? forced_tile : tile_choice<A8>(m, n, k, ol.idx == nullptr);
    switch (tile) {
    case 256256:
        return launch_pp<A8>(x, sx, q, scales, zeros, ol, y, m, n, k, stream);
    case 256128:
        return launch_dma<4, 256, 128, A8>(x, sx, q, scales, zeros, ol, y, m, n, k, stream);
    case 256064:
        return launch_dma<4, 256, 64, A8>(x, sx, q, scales, zeros, ol, y, m, n, k, stream);
    case 128128:
        if constexpr (!A8)
            return launch_dma<4, 128, 128, A8>(x, sx, q, scales, zeros, ol, y, m, n, k, stream);
        [[fallthrough]];
    default:
        return launch_dma<4, 128, 64, A8>(x, sx, q, scales, zeros, ol, y, m, n, k, stream);
    }
}

} // namespace

int mfma_tile_choice(int64_t m, int64_t n, int64_t k)
{
    return tile_choice<false>(m, n, k);
}

int w8a8_tile_choice(int64_t m, int64_t n, int64_t k)
{
    return tile_choice<true>(m, n, k);
}

hipError_t launch_mfma_gemm(const uint16_t *x, const int8_t *q, const uint16_t *scales,
                            const int8_t *zeros, OutlierList ol, uint16_t *y, int64_t m, int64_t n,
                            int64_t k, hipStream_t stream)
{
    return launch_tiles<false>(x, nullptr, q, scales, zeros, ol, y, m, n, k, stream);
}

hipError_t launch_mfma_gemm_tile(int tile, const uint16_t *x, const int8_t *q, const uint16_t *scales,
                                 const int8_t *zeros, OutlierList ol, uint16_t *y, int64_t m, int64_t n,
                                 int64_t k, hipStream_t stream)
{
    if (tile != 256256 && tile != 256128 && tile != 256064 && tile != 128128 && tile != 128064)
        return hipErrorInvalidValue;
    if (tile == 256256 && k > kPingPongMaxK)
        return hipErrorInvalidValue;
    return launch_tiles<false>(x, nullptr, q, scales, zeros, ol, y, m, n, k, stream, tile);
}

hipError_t launch_w8a8_gemm_tile(int tile, const int8_t *qx, const uint16_t *sx, const int8_t *q,
                                 const uint16_t *scales, uint16_t *y, int64_t m, int64_t n, int64_t k,
                                 hipStream_t stream)
{
    if (tile != 256256 && tile != 256128 && tile != 256064 && tile != 128064)
        return hipErrorInvalidValue;
    return launch_tiles<true>(qx, sx, q, scales, nullptr, OutlierList{nullptr, nullptr, 0}, y, m, n, k, stream,
                              tile);
}

hipError_t launch_w8a8_gemm(const int8_t *qx, const uint16_t *sx, const int8_t *q,
                            const uint16_t *scales, uint16_t *y, int64_t m, int64_t n, int64_t k,
                            hipStream_t stream)
{
    return launch_tiles<true>(qx, sx, q, scales, nullptr, OutlierList{nullptr, nullptr, 0}, y, m, n, k, stream);
}

} // namespace qw

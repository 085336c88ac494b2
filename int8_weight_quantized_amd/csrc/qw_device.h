// qw_device.h -- device helpers shared by the gfx950 kernels of libqw.
//
// Wave size is 64 on CDNA; every helper below assumes it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qw {

constexpr int kWave = 64;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// int8 -> fp16, exact.
//
// The int8 code q (two's complement) is turned into the offset-binary byte
// u = q + 128 by flipping the top bit, then placed under the binary16
// exponent pattern 0x64 so that the half reads 1024 + u exactly; one packed
// fp16 subtraction of 1152 then leaves q exactly (all values involved are
// integers below 2048, representable in binary16).  Per 4 codes: one XOR,
// two byte permutes, two packed subtracts.
// ---------------------------------------------------------------------------
//
// Subtracting 1152 + z instead of 1152 yields q - z, the asymmetric
// dequantization's integer part, at no extra cost: q - z lies in [-255,
// 255], and every operand and result of the subtraction is an integer
// below 2048, so it is exact in fp16.  `bias` holds 1152 + z in both halves
// (zero_point_bias below).
__device__ __forceinline__ void i8x4_to_half2x2(uint32_t codes, half2_t &lo, half2_t &hi,
                                                half2_t bias = (half2_t){(_Float16)1152.0f, (_Float16)1152.0f})
{
    const uint32_t u = codes ^ 0x80808080u;
    // v_perm_b32: bytes 0..3 come from the second operand, 4..7 from the first.
    const uint32_t plo = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u); // [u0,64,u1,64]
    const uint32_t phi = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u); // [u2,64,u3,64]
    lo = __builtin_bit_cast(half2_t, plo) - bias;
    hi = __builtin_bit_cast(half2_t, phi) - bias;
}

// The cast bias for zero point z (z = 0: the plain int8 -> fp16 cast).
__device__ __forceinline__ half2_t zero_point_bias(int z)
{
    const _Float16 b = (_Float16)(float)(1152 + z); // exact: 1024 <= 1152 + z <= 1279
    return (half2_t){b, b};
}

// 16 int8 codes (one 16-byte load) -> 8 packed half2 values, in k order.
__device__ __forceinline__ void i8x16_to_half2x8(const u32x4_t v, half2_t h[8],
                                                 half2_t bias = (half2_t){(_Float16)1152.0f, (_Float16)1152.0f})
{
    i8x4_to_half2x2(v.x, h[0], h[1], bias);
    i8x4_to_half2x2(v.y, h[2], h[3], bias);
    i8x4_to_half2x2(v.z, h[4], h[5], bias);
    i8x4_to_half2x2(v.w, h[6], h[7], bias);
}

// 8 int8 codes -> one half8 MFMA operand, in k order.
__device__ __forceinline__ half8_t i8x8_to_half8(uint32_t a, uint32_t b,
                                                 half2_t bias = (half2_t){(_Float16)1152.0f, (_Float16)1152.0f})
{
    half2_t h0, h1, h2, h3;
    i8x4_to_half2x2(a, h0, h1, bias);
    i8x4_to_half2x2(b, h2, h3, bias);
    half8_t r = {h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
    return r;
}

// Reinterpret a 32-bit value as a pair of halves.  Takes the value by copy:
// clang's __builtin_bit_cast applied directly to an ext-vector component
// (e.g. v.y) reads component 0 instead, so never bit-cast `v.y` in place.
__device__ __forceinline__ half2_t as_half2(uint32_t bits)
{
    return __builtin_bit_cast(half2_t, bits);
}

// fp32 dot of two fp16 pairs accumulated into fp32 (v_dot2_f32_f16).
__device__ __forceinline__ float dot2(half2_t a, half2_t b, float c)
{
    return __builtin_amdgcn_fdot2(a, b, c, false);
}

// fp32 -> binary16 bits, round to nearest even (v_cvt_f16_f32 in the
// default rounding mode).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float v)
{
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b)
{
    return (float)__builtin_bit_cast(_Float16, b);
}

// ---------------------------------------------------------------------------
// Cross-lane helpers (wave64).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float shfl_xor_f32(float v, int mask)
{
    const int lane = __lane_id();
    const int src = lane ^ mask;
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, v)));
}

__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v, int mask)
{
    const int lane = __lane_id();
    const int src = lane ^ mask;
    return (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, (int)v);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        const uint32_t o = shfl_xor_u32(v, d);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        const uint32_t o = shfl_xor_u32(v, d);
        v = o < v ? o : v;
    }
    return v;
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        v += shfl_xor_u32(v, d);
    return v;
}

// Transposing butterfly reduction of R per-lane partial sums across the 64
// lanes of a wave (R a power of two, R <= 64).  At each step a lane keeps
// one half of its values and receives the partner's copy of that half, so
// R values cost about R shuffles instead of 6 R.  On return, lane l holds
// the full sum of value index `butterfly_index<R>(l)` in v[0] whenever
// (l & (64 / R - 1)) == 0.
template <int R>
__device__ __forceinline__ void butterfly_reduce(float (&v)[R])
{
    static_assert(R >= 1 && R <= 64 && (R & (R - 1)) == 0, "R must be a power of two <= 64");
    const int lane = __lane_id();
    int width = R;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        if (width > 1) {
            const int half = width >> 1;
            const bool upper = (lane & d) != 0;
#pragma unroll
            for (int j = 0; j < R / 2; ++j) {
                if (j < half) {
                    const float send = upper ? v[j] : v[j + half];
                    const float keep = upper ? v[j + half] : v[j];
                    v[j] = keep + shfl_xor_f32(send, d);
                }
            }
            width = half;
        } else {
            v[0] += shfl_xor_f32(v[0], d);
        }
    }
}

template <int R>
__device__ __forceinline__ int butterfly_index(int lane)
{
    int idx = 0;
    int width = R;
#pragma unroll
    for (int d = 32; d >= 1 && width > 1; d >>= 1) {
        width >>= 1;
        if (lane & d)
            idx += width;
    }
    return idx;
}

} // namespace qw

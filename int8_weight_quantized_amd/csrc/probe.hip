// probe.hip -- two measurement aids that put the GEMM figures in context.
//
// qw_probe_stream_read: the plainest kernel that reads a buffer once from
// HBM, with the same access shape the decode GEMV uses (16-byte
// nontemporal loads, one contiguous 1 KiB per wave instruction, several
// loads in flight per wave).  Its rate on a cold buffer of the weight's
// size is the practical ceiling a weight-streaming GEMV can reach on the
// box, next to the 8 TB/s of the data sheet.  Nothing is written unless
// the folded value of a wave's bytes happens to equal `magic` (the caller
// passes a value that makes this practically never happen); the
// comparison only keeps the loads from being optimised away.
//
// qw_probe_shader_clock: one wave reads the shader-clock counter
// (s_memtime) and the 100 MHz constant clock (s_memrealtime) across a
// spin of about 20 us and stores both deltas, from which the host
// derives the clock the compute units ran at right then.  Enqueued right
// after a timed loop it reads the clock the loop left the chip at.
#include "qw_device.h"
#include "qw_internal.h"

namespace qw {
namespace {

constexpr int kReadUnroll = 8;    // 1 KiB loads in flight per wave per round
constexpr int kReadWavesPerCu = 8; // measured best with 8 loads in flight

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t *__restrict__ p, int64_t chunks,
                                                          int64_t waves, uint32_t magic,
                                                          uint32_t *__restrict__ sink)
{
    const int lane = __lane_id();
    const int64_t w = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    if (w >= waves)
        return;
    uint32_t acc = 0;
    // round r covers chunks [r * waves * U, (r + 1) * waves * U): wave w takes
    // chunks w, w + waves, ..., so the chip reads one compact window at a time
    for (int64_t base = 0; base < chunks; base += waves * kReadUnroll) {
        u32x4_t v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) {
            const int64_t c = base + u * waves + w;
            v[u] = c < chunks ? __builtin_nontemporal_load(p + c * kWave + lane) : (u32x4_t){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == magic)
        sink[0] = acc;
}

__global__ __launch_bounds__(64) void shader_clock_kernel(uint64_t ticks, uint64_t *__restrict__ out)
{
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    uint64_t r1 = r0;
    // bounded by the constant clock: ends after `ticks` of 100 MHz
    while (r1 - r0 < ticks) {
        __builtin_amdgcn_s_sleep(1);
        r1 = __builtin_amdgcn_s_memrealtime();
    }
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    if (threadIdx.x == 0) {
        out[0] = c1 - c0;
        out[1] = r1 - r0;
    }
}

} // namespace

hipError_t launch_stream_read(const void *p, int64_t bytes, uint32_t magic, uint32_t *sink, hipStream_t stream)
{
    const int64_t chunks = bytes / 1024;
    if (chunks == 0)
        return hipSuccess;
    int64_t waves = (int64_t)device_cu_count() * kReadWavesPerCu;
    // equal rounds for every wave
    const int64_t rounds = (chunks + waves * kReadUnroll - 1) / (waves * kReadUnroll);
    waves = (chunks + rounds * kReadUnroll - 1) / (rounds * kReadUnroll);
    const int64_t blocks = (waves + 3) / 4;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const u32x4_t *>(p), chunks, waves, magic, sink);
    return hipGetLastError();
}

hipError_t launch_shader_clock(uint64_t *out, hipStream_t stream)
{
    hipLaunchKernelGGL(shader_clock_kernel, dim3(1), dim3(64), 0, stream, (uint64_t)2000, out);
    return hipGetLastError();
}

} // namespace qw

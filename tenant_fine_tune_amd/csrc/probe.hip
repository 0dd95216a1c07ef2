// Measurement probes: the device's practical streaming-read rate and dense
// bf16 MFMA rate, measured beside the method's kernels so that their
// rooflines can be read against what this chip sustains as well as against
// its published peaks.  Neither computes anything of the method.
//
//  probe_read: reads a buffer once with 16-byte streaming loads, one 1 KB
//    contiguous run per wave instruction, wave g reading the 8 KB of runs
//    8g .. 8g + 7 with all eight loads in flight (the access pattern of the
//    decode kernels, where a wave streams one 8 KB row), and folds the data
//    into one XOR word per wave so that no load can be dropped.
//  probe_mfma: each wave runs `iters` rounds of eight independent
//    v_mfma_f32_32x32x16_bf16 on register operands (no memory traffic) and
//    writes one fp32 word per wave: the sum of lane 0's first accumulator
//    element over the eight accumulators, which is 8 * 16 * iters * a * b for
//    operands that are all a (A) and b (B).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bd_device.h"
#include "bd_launch.h"

namespace bd {
namespace {

constexpr int kProbeWaves = 4;    // waves per workgroup
constexpr int kProbeRuns = 8;     // 1 KB runs per wave

__global__ __launch_bounds__(64 * kProbeWaves) void probe_read(const uint8_t *__restrict__ src, int64_t bytes,
                                                               uint32_t *__restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const int64_t g = (int64_t)blockIdx.x * kProbeWaves + (threadIdx.x >> 6);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, bytes);
    uint4 v[kProbeRuns];
#pragma unroll
    for (int i = 0; i < kProbeRuns; ++i) {
        const int64_t off = (g * kProbeRuns + i) * 1024 + lane * 16;
        // past the end: the out-of-range lane offset (reads zero)
        const uint32_t o = off + 16 <= bytes ? (uint32_t)off : kInvalidOffset;
        v[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, kStream));
    }
    uint32_t h = 0;
#pragma unroll
    for (int i = 0; i < kProbeRuns; ++i)
        h ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    for (int o = 32; o > 0; o >>= 1)
        h ^= __shfl_xor(h, o);
    if (lane == 0)
        sink[g] = h;
}

__global__ __launch_bounds__(64 * kProbeWaves) void probe_mfma(int32_t iters, float a, float b,
                                                               uint32_t *__restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const int64_t g = (int64_t)blockIdx.x * kProbeWaves + (threadIdx.x >> 6);
    bf16x8 A, B;
    const uint16_t ab = (uint16_t)(__float_as_uint(a) >> 16), bb = (uint16_t)(__float_as_uint(b) >> 16);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        A[e] = __builtin_bit_cast(__bf16, ab);
        B[e] = __builtin_bit_cast(__bf16, bb);
    }
    f32x16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
            acc[i][e] = 0.0f;
        asm volatile("" : "+a"(acc[i]));
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, acc[i], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        s += acc[i][0];
    if (lane == 0)
        sink[g] = __float_as_uint(s);
}

}  // namespace

int64_t probe_read_sink_words(int64_t bytes)
{
    const int64_t runs = (bytes + 1023) / 1024;
    const int64_t blocks = (runs + kProbeRuns * kProbeWaves - 1) / (kProbeRuns * kProbeWaves);
    return blocks * kProbeWaves;
}

hipError_t launch_probe_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t s)
{
    const int64_t blocks = probe_read_sink_words(bytes) / kProbeWaves;
    hipLaunchKernelGGL(probe_read, dim3((unsigned)blocks), dim3(64 * kProbeWaves), 0, s,
                       static_cast<const uint8_t *>(src), bytes, sink);
    return hipGetLastError();
}

hipError_t launch_probe_mfma(int32_t blocks, int32_t iters, float a, float b, uint32_t *sink, hipStream_t s)
{
    hipLaunchKernelGGL(probe_mfma, dim3((unsigned)blocks), dim3(64 * kProbeWaves), 0, s, iters, a, b, sink);
    return hipGetLastError();
}

}  // namespace bd

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
//  probe_lds: the LDS rates a kernel's staging is built from.  One
//    workgroup of 16 waves per CU (it declares 96 KB of LDS, so no second
//    one fits) fills 64 KB of LDS with word i = i * 0x9E3779B1, then each
//    wave issues iters x 8 conflict-free LDS operations, each moving one
//    contiguous block: mode 0 ds_read_b128 of 1 KB block (u * stride + w) mod
//    64, mode 1 ds_read_b64 of 512-byte block (u * stride + w) mod 128, mode 2
//    ds_write_b128 of 1 KB into block 4w + u mod 4 of the wave's own 4 KB,
//    mode 3 a direct-to-LDS copy of 1 KB block (u * stride + w) mod
//    (src_bytes / 1 KB) of `src` into that same block (u = 8 it + j, the
//    operation's index; w the wave).  The shader clock between two workgroup
//    barriers around the loop (the copies drained) goes to cycles[block];
//    sink[block * 16 + w] is the XOR of every word the wave read (modes 0, 1)
//    or of its 4 KB after the loop (modes 2, 3), so no operation can be
//    dropped.  Mode 2 writes, for lane l, the words u * 0x9E3779B1 + l,
//    (u << 8) ^ l, u + l * 0x01000193 and ~(u ^ (l << 16)).
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

constexpr int kLdsWaves = 16;
constexpr int kLdsWords = 16384;          // 64 KB used
constexpr int kLdsAsk = 24576;            // words declared: 96 KB, one workgroup per CU

template <int MODE>
__global__ __launch_bounds__(64 * kLdsWaves) void probe_lds(int32_t iters, uint32_t stride,
                                                            const uint8_t *__restrict__ src, uint32_t src_blocks,
                                                            uint32_t *__restrict__ sink, uint64_t *__restrict__ cycles)
{
    __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsAsk];
    const int tid = threadIdx.x, lane = tid & 63;
    const uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane(tid >> 6);
    for (int i = tid; i < kLdsWords; i += 64 * kLdsWaves)
        lds[i] = (uint32_t)i * 0x9E3779B1u;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, MODE == 3 ? (int64_t)src_blocks * 1024 : 0);
    uint32_t acc = 0;
    __syncthreads();
    const uint64_t t0 = __builtin_readcyclecounter();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t u = (uint32_t)(it * 8 + j);
            if constexpr (MODE == 0) {
                const uint32_t blk = (u * stride + wave) & 63u;
                const uint4 v = *reinterpret_cast<const uint4 *>(&lds[blk * 256 + lane * 4]);
                acc ^= v.x ^ v.y ^ v.z ^ v.w;
            } else if constexpr (MODE == 1) {
                const uint32_t blk = (u * stride + wave) & 127u;
                const uint2 v = *reinterpret_cast<const uint2 *>(&lds[blk * 128 + lane * 2]);
                acc ^= v.x ^ v.y;
            } else if constexpr (MODE == 2) {
                const uint32_t blk = wave * 4 + (u & 3u);
                *reinterpret_cast<uint4 *>(&lds[blk * 256 + lane * 4]) =
                    make_uint4(u * 0x9E3779B1u + lane, (u << 8) ^ lane, u + lane * 0x01000193u, ~(u ^ (lane << 16)));
                // every store is issued (a later one to the same block does not
                // make it dead to the compiler)
                asm volatile("" ::: "memory");
            } else {
                const uint32_t blk = wave * 4 + (u & 3u);
                const uint32_t sb = (u * stride + wave) & (src_blocks - 1);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(&lds[blk * 256]), 16, (uint32_t)(16 * lane),
                                                         sb * 1024u, 0, 0);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const uint64_t t1 = __builtin_readcyclecounter();
    if constexpr (MODE >= 2) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4 v = *reinterpret_cast<const uint4 *>(&lds[(wave * 4 + c) * 256 + lane * 4]);
            acc ^= v.x ^ v.y ^ v.z ^ v.w;
        }
    }
    for (int o = 32; o > 0; o >>= 1)
        acc ^= __shfl_xor(acc, o);
    if (lane == 0)
        sink[(int64_t)blockIdx.x * kLdsWaves + wave] = acc;
    if (tid == 0)
        cycles[blockIdx.x] = t1 - t0;
}

}  // namespace

hipError_t launch_probe_lds(int32_t blocks, int32_t iters, int32_t mode, int32_t stride, const void *src,
                            int64_t src_bytes, uint32_t *sink, uint64_t *cycles, hipStream_t s)
{
    const dim3 grid((unsigned)blocks), block(64 * kLdsWaves);
    const uint8_t *sp = static_cast<const uint8_t *>(src);
    const uint32_t nb = mode == 3 ? (uint32_t)(src_bytes >> 10) : 1;
    switch (mode) {
    case 0: hipLaunchKernelGGL(probe_lds<0>, grid, block, 0, s, iters, (uint32_t)stride, sp, nb, sink, cycles); break;
    case 1: hipLaunchKernelGGL(probe_lds<1>, grid, block, 0, s, iters, (uint32_t)stride, sp, nb, sink, cycles); break;
    case 2: hipLaunchKernelGGL(probe_lds<2>, grid, block, 0, s, iters, (uint32_t)stride, sp, nb, sink, cycles); break;
    default: hipLaunchKernelGGL(probe_lds<3>, grid, block, 0, s, iters, (uint32_t)stride, sp, nb, sink, cycles); break;
    }
    return hipGetLastError();
}

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

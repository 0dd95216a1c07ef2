// Compress kernels: Delta, sign, bit packing and alpha.
//
// "BitDelta: Serving 14 Zen Models from One GPU Cluster", section
// "Mathematical Foundation": Delta = W_ft - W_base is reduced to one sign bit
// per weight plus one scale alpha = mean |Delta|; section "Infrastructure
// Details": signs stored 8 per byte, alpha as fp32 per output row.
//
// One workgroup of 256 threads per row.  Thread t owns the 8-column groups
// g = t, t+256, t+512, ... of the row, so partial sum k of the fixed
// summation order is exactly thread k's running fp64 sum; the halving tree
// p[k] += p[k+s] (s = 128 ... 1) then runs in LDS.  HBM traffic is one read
// of W_base (2 B/weight) and W_ft (4 or 2 B/weight) and one write of the sign
// byte (1/8 B/weight): the kernel is bandwidth-bound.
#include "bd_device.h"
#include "bd_launch.h"

namespace bd {
namespace {

constexpr int kThreads = 256;

// The halving tree p[k] += p[k + s], s = 128, 64, ..., 1, over the 256
// threads' values (thread k holds p[k]); returns p[0] in every thread of
// wave 0.  Steps s >= 64 cross waves and go through LDS; steps s <= 32 stay
// in wave 0 and use lane shuffles.  Same additions, same order, as the tree
// written out in full.
__device__ __forceinline__ double halving_tree(double v, double *sp)
{
    const int t = threadIdx.x;
    if (t >= 128)
        sp[t - 128] = v;                    // p[128..255]
    __syncthreads();
    if (t < 128) {
        v = v + sp[t];                      // s = 128
        if (t >= 64)
            sp[128 + t - 64] = v;           // p[64..127]
    }
    __syncthreads();
    if (t < 64) {
        v = v + sp[128 + t];                // s = 64
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1)
            v = v + __shfl_down(v, s, 64);  // lanes >= 64 - s read junk, never used by lane 0's chain
    }
    return v;
}

template <bool FT_F32>
__device__ __forceinline__ void load_group(const uint4 *wb, const void *w_ft, int64_t r, int64_t C, int64_t g,
                                           uint4 &b, float (&ft)[8])
{
    b = ld_stream16(wb + g);
    if constexpr (FT_F32) {
        const uint4 *f = reinterpret_cast<const uint4 *>(static_cast<const float *>(w_ft) + r * C);
        const uint4 a0 = ld_stream16(f + 2 * g), a1 = ld_stream16(f + 2 * g + 1);
        ft[0] = __uint_as_float(a0.x); ft[1] = __uint_as_float(a0.y);
        ft[2] = __uint_as_float(a0.z); ft[3] = __uint_as_float(a0.w);
        ft[4] = __uint_as_float(a1.x); ft[5] = __uint_as_float(a1.y);
        ft[6] = __uint_as_float(a1.z); ft[7] = __uint_as_float(a1.w);
    } else {
        const uint4 f = ld_stream16(reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(w_ft) + r * C) + g);
        ft[0] = lo_f32(f.x); ft[1] = hi_f32(f.x); ft[2] = lo_f32(f.y); ft[3] = hi_f32(f.y);
        ft[4] = lo_f32(f.z); ft[5] = hi_f32(f.z); ft[6] = lo_f32(f.w); ft[7] = hi_f32(f.w);
    }
}

// Sign byte of one group; adds the 8 |Delta| to p in column order.
__device__ __forceinline__ uint8_t sign_group(const uint4 &b, const float (&ft)[8], double &p)
{
    const float wf[8] = {lo_f32(b.x), hi_f32(b.x), lo_f32(b.y), hi_f32(b.y),
                         lo_f32(b.z), hi_f32(b.z), lo_f32(b.w), hi_f32(b.w)};
    uint32_t byte = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float d = ft[i] - wf[i];
        byte |= (d >= 0.0f ? 1u : 0u) << i;
        p = p + (double)fabsf(d);
    }
    return (uint8_t)byte;
}

template <bool FT_F32, bool PER_MATRIX>
__global__ __launch_bounds__(kThreads) void compress_rows(const uint16_t *__restrict__ w_base,
                                                          const void *__restrict__ w_ft, int64_t C,
                                                          uint8_t *__restrict__ signs,
                                                          float *__restrict__ alpha,
                                                          double *__restrict__ row_sums)
{
    __shared__ double sp[192];
    const int64_t r = blockIdx.x;
    const int64_t G = C >> 3;
    const uint4 *wb = reinterpret_cast<const uint4 *>(w_base + r * C);
    uint8_t *srow = signs + r * G;
    double p = 0.0;
    int64_t g = threadIdx.x;
    // four groups per pass, all loads issued before the first subtraction
    for (; g + 3 * kThreads < G; g += 4 * kThreads) {
        uint4 b[4];
        float ft[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            load_group<FT_F32>(wb, w_ft, r, C, g + u * kThreads, b[u], ft[u]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            srow[g + u * kThreads] = sign_group(b[u], ft[u], p);
    }
    if (g + kThreads < G) {
        uint4 b[2];
        float ft[2][8];
        load_group<FT_F32>(wb, w_ft, r, C, g, b[0], ft[0]);
        load_group<FT_F32>(wb, w_ft, r, C, g + kThreads, b[1], ft[1]);
        srow[g] = sign_group(b[0], ft[0], p);
        srow[g + kThreads] = sign_group(b[1], ft[1], p);
        g += 2 * kThreads;
    }
    if (g < G) {
        uint4 b;
        float ft[8];
        load_group<FT_F32>(wb, w_ft, r, C, g, b, ft);
        srow[g] = sign_group(b, ft, p);
    }
    const double S = halving_tree(p, sp);
    if (threadIdx.x == 0) {
        if constexpr (PER_MATRIX)
            row_sums[r] = S;
        else
            alpha[r] = (float)(S / (double)C);
    }
}

// Per-matrix alpha: row r's sum goes into partial r mod 256 (rows in
// increasing order), then the same halving tree; one fp64 divide and one
// rounding to fp32.  Loads go out 16 rows at a time ahead of the adds.
__global__ __launch_bounds__(kThreads) void alpha_matrix_finish(const double *__restrict__ row_sums,
                                                                int64_t R, int64_t C,
                                                                float *__restrict__ alpha)
{
    __shared__ double sp[192];
    double q = 0.0;
    int64_t r = threadIdx.x;
    for (; r + 15 * kThreads < R; r += 16 * kThreads) {
        double v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
            v[u] = row_sums[r + u * kThreads];
#pragma unroll
        for (int u = 0; u < 16; ++u)
            q = q + v[u];
    }
    for (; r < R; r += kThreads)
        q = q + row_sums[r];
    const double T = halving_tree(q, sp);
    if (threadIdx.x == 0)
        alpha[0] = (float)(T / ((double)R * (double)C));
}

}  // namespace

hipError_t launch_compress(const uint16_t *w_base, const void *w_ft, bool ft_f32, int64_t d_out,
                           int64_t d_in, bool per_matrix, uint8_t *signs, float *alpha,
                           double *row_sums, hipStream_t s)
{
    const dim3 grid((unsigned)d_out), block(kThreads);
    if (ft_f32) {
        if (per_matrix)
            hipLaunchKernelGGL((compress_rows<true, true>), grid, block, 0, s, w_base, w_ft, d_in, signs, alpha, row_sums);
        else
            hipLaunchKernelGGL((compress_rows<true, false>), grid, block, 0, s, w_base, w_ft, d_in, signs, alpha, row_sums);
    } else {
        if (per_matrix)
            hipLaunchKernelGGL((compress_rows<false, true>), grid, block, 0, s, w_base, w_ft, d_in, signs, alpha, row_sums);
        else
            hipLaunchKernelGGL((compress_rows<false, false>), grid, block, 0, s, w_base, w_ft, d_in, signs, alpha, row_sums);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !per_matrix)
        return e;
    hipLaunchKernelGGL(alpha_matrix_finish, dim3(1), block, 0, s, row_sums, d_out, d_in, alpha);
    return hipGetLastError();
}

}  // namespace bd

// Decode kernel: fused BitDelta linear for m <= 16 tokens, no MFMA.
//
// "BitDelta: Serving 14 Zen Models from One GPU Cluster", section "Serving
// Architecture": the fused kernel reads the base weights and the packed
// delta bits together and builds the effective weight in registers, never
// writing W_eff to HBM (the conceptual fused_bitdelta_linear sketch gives the
// semantics y = x (W_base + alpha * unpack(signs))^T).
//
// At m <= 16 the layer is bound by HBM bandwidth (about 1 to 15 flop per
// byte of W_base + signs), so this kernel is a streaming GEMV on the vector
// ALUs:
//  - a wave owns RW output rows; its 64 lanes walk a row 512 columns at a
//    time, each lane one 16-byte load of W_base (8 weights) and the matching
//    sign byte, so every load instruction is fully coalesced;
//  - W_eff is formed in VGPRs: fp32 add of +-alpha, one v_cvt_pk_bf16_f32 per
//    pair, giving packed bf16 pairs;
//  - the activations of a slab of columns are staged in LDS once per
//    workgroup and read as 16-byte vectors; each packed W_eff pair is
//    multiplied into every token with v_dot2_f32_bf16 (fp32 accumulate);
//  - at the end each (row, token) partial is reduced across the 64 lanes.
#include "bd_device.h"
#include "bd_launch.h"

namespace bd {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kLdsBytes = 64 * 1024;

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// MT: token tile (tokens >= m are zero in LDS and never stored).
// RW: rows per wave.
template <int MT, int RW, bool PER_MATRIX>
__global__ __launch_bounds__(kThreads) void gemv_rows(const uint16_t *__restrict__ x, int m,
                                                      const uint16_t *__restrict__ w_base,
                                                      const uint8_t *__restrict__ signs,
                                                      const float *__restrict__ alpha,
                                                      int64_t R, int64_t C,
                                                      uint16_t *__restrict__ y)
{
    constexpr int SLAB = kLdsBytes / (16 * MT);  // 8-column groups per slab
    extern __shared__ uint4 xs[];                // [MT][SLAB] groups of 8 bf16
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t row0 = ((int64_t)blockIdx.x * kWaves + wave) * RW;
    const int64_t G = C >> 3;

    float acc[RW][MT];
    float a[RW];
    bool valid[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        valid[r] = row0 + r < R;
        a[r] = valid[r] ? (PER_MATRIX ? alpha[0] : alpha[row0 + r]) : 0.0f;
#pragma unroll
        for (int t = 0; t < MT; ++t)
            acc[r][t] = 0.0f;
    }

    const uint4 *x4 = reinterpret_cast<const uint4 *>(x);
    for (int64_t s0 = 0; s0 < G; s0 += SLAB) {
        const int sg = (int)min((int64_t)SLAB, G - s0);
        __syncthreads();
        for (int i = threadIdx.x; i < MT * sg; i += kThreads) {
            const int t = i / sg, g = i - t * sg;
            xs[t * SLAB + g] = t < m ? x4[(int64_t)t * G + s0 + g] : make_uint4(0, 0, 0, 0);
        }
        __syncthreads();
        for (int g = lane; g < sg; g += 64) {
            uint4 w[RW];
            uint32_t sb[RW];
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const int64_t off = (row0 + r) * G + s0 + g;
                w[r] = valid[r] ? reinterpret_cast<const uint4 *>(w_base)[off] : make_uint4(0, 0, 0, 0);
                sb[r] = valid[r] ? (uint32_t)signs[off] : 0u;
            }
            uint4 e[RW];
#pragma unroll
            for (int r = 0; r < RW; ++r)
                e[r] = weff_group(w[r], sb[r], a[r]);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const uint4 xv = xs[t * SLAB + g];
#pragma unroll
                for (int r = 0; r < RW; ++r) {
                    float c = acc[r][t];
                    c = dot2(e[r].x, xv.x, c);
                    c = dot2(e[r].y, xv.y, c);
                    c = dot2(e[r].z, xv.z, c);
                    c = dot2(e[r].w, xv.w, c);
                    acc[r][t] = c;
                }
            }
        }
    }

#pragma unroll
    for (int r = 0; r < RW; ++r) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const float v = wave_sum(acc[r][t]);
            if (lane == 0 && valid[r] && t < m)
                y[(int64_t)t * R + row0 + r] = to_bf16(v);
        }
    }
}

template <int MT, int RW>
hipError_t launch_tile(const uint16_t *x, int m, const uint16_t *w_base, const uint8_t *signs,
                       const float *alpha, bool per_matrix, int64_t d_out, int64_t d_in,
                       uint16_t *y, hipStream_t s)
{
    const int64_t rows_per_block = (int64_t)kWaves * RW;
    const dim3 grid((unsigned)((d_out + rows_per_block - 1) / rows_per_block)), block(kThreads);
    if (per_matrix)
        hipLaunchKernelGGL((gemv_rows<MT, RW, true>), grid, block, kLdsBytes, s, x, m, w_base, signs, alpha, d_out, d_in, y);
    else
        hipLaunchKernelGGL((gemv_rows<MT, RW, false>), grid, block, kLdsBytes, s, x, m, w_base, signs, alpha, d_out, d_in, y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const uint16_t *x, int m, const uint16_t *w_base, const uint8_t *signs,
                       const float *alpha, bool per_matrix, int64_t d_out, int64_t d_in,
                       uint16_t *y, hipStream_t s)
{
    if (m <= 1)
        return launch_tile<1, 4>(x, m, w_base, signs, alpha, per_matrix, d_out, d_in, y, s);
    if (m <= 2)
        return launch_tile<2, 4>(x, m, w_base, signs, alpha, per_matrix, d_out, d_in, y, s);
    if (m <= 4)
        return launch_tile<4, 2>(x, m, w_base, signs, alpha, per_matrix, d_out, d_in, y, s);
    if (m <= 8)
        return launch_tile<8, 2>(x, m, w_base, signs, alpha, per_matrix, d_out, d_in, y, s);
    return launch_tile<16, 2>(x, m, w_base, signs, alpha, per_matrix, d_out, d_in, y, s);
}

}  // namespace bd

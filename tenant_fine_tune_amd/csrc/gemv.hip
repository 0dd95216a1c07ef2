// Decode kernel: fused BitDelta linear for m <= 16 tokens, no MFMA.
//
// "BitDelta: Serving 14 Zen Models from One GPU Cluster", section "Serving
// Architecture": the fused kernel reads the base weights and the packed
// delta bits together and builds the effective weight in registers, never
// writing W_eff to HBM (the conceptual fused_bitdelta_linear sketch gives the
// semantics y = x (W_base + alpha * unpack(signs))^T).
//
// At m <= 16 the layer is bound by HBM bandwidth (1 to 15 flop per byte of
// W_base + signs), so this is a streaming GEMV on the vector ALUs whose job
// is to keep enough bytes in flight:
//  - a wave owns RW output rows and walks them 512 columns per step: lane l
//    loads the 16 bytes of columns 8l..8l+7 of each row (every load
//    instruction covers 1 KB of contiguous W_base) plus their sign byte;
//  - a ring of D register stages keeps the next D steps' loads outstanding;
//    the loop is split into a steady part (consume a stage, refill it D steps
//    ahead) and a drain, with every load address clamped into the tensor, so
//    no load sits under a branch and the compiler's wait counters stay exact
//    (a branch around a load makes it wait for all loads at the join);
//  - W_eff is formed in VGPRs (fp32 add of +-alpha, v_cvt_pk_bf16_f32 per
//    pair) and each packed pair is multiplied into every token with
//    v_dot2_f32_bf16 (fp32 accumulate);
//  - m <= 4: the activations ride in the same ring (16-byte loads that hit
//    L1/L2: x is at most 32 KB per row and shared by every wave);
//    m in 5..16: they are staged per slab in LDS and read as 16-byte vectors,
//    and each wave owns 4 rows to amortise those reads;
//  - the RW * MT per-lane partial sums are reduced across the wave by a
//    reduce-scatter (each halving step exchanges half of the values).
#include <algorithm>

#include "bd_device.h"
#include "bd_launch.h"

namespace bd {
namespace {

constexpr int kMaxLdsBytes = 128 * 1024;

// One halving step of a reduce-scatter: lanes whose `MASK` bit is clear keep
// values [0, HALF), the others keep [HALF, 2*HALF), each adding its partner's
// copy; the kept values end up in v[0 .. HALF).
template <int HALF, int MASK, int N>
__device__ __forceinline__ void halve(float (&v)[N], int lane)
{
    if constexpr (HALF >= 1) {
        const bool low = (lane & MASK) == 0;
#pragma unroll
        for (int j = 0; j < HALF; ++j) {
            const float send = low ? v[j + HALF] : v[j];
            const float keep = low ? v[j] : v[j + HALF];
            v[j] = keep + __shfl_xor(send, MASK, 64);
        }
        halve<HALF / 2, MASK / 2>(v, lane);
    }
}

template <int N>
constexpr int log2i() { return N <= 1 ? 0 : 1 + log2i<N / 2>(); }

// Reduce-scatter of N = 2^k values over the 64 lanes of a wave.  Returns, in
// every lane, the full sum of value index (lane >> (6 - k)).
template <int N>
__device__ __forceinline__ float wave_reduce_scatter(float (&v)[N])
{
    static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "N must be a power of two <= 64");
    const int lane = threadIdx.x & 63;
    halve<N / 2, 32>(v, lane);
    float s = v[0];
#pragma unroll
    for (int mask = 32 >> log2i<N>(); mask >= 1; mask >>= 1)
        s += __shfl_xor(s, mask, 64);
    return s;
}

template <int RW, int MT>
__device__ __forceinline__ void store_rows(float (&acc)[RW * MT], int64_t row0, int64_t R, int m,
                                           uint16_t *__restrict__ y)
{
    constexpr int N = RW * MT;
    constexpr int kbits = log2i<N>();
    const int lane = threadIdx.x & 63;
    const float v = wave_reduce_scatter<N>(acc);
    const int idx = lane >> (6 - kbits);
    if ((lane & ((1 << (6 - kbits)) - 1)) == 0) {
        const int r = idx / MT, t = idx - r * MT;
        if (row0 + r < R && t < m)
            y[(int64_t)t * R + row0 + r] = to_bf16(v);
    }
}

template <int RW, bool PER_MATRIX>
struct Rows {
    const uint4 *w[RW];
    const uint8_t *s[RW];
    float a[RW];
    __device__ __forceinline__ Rows(const uint16_t *w_base, const uint8_t *signs, const float *alpha,
                                    int64_t row0, int64_t R, int64_t C)
    {
        const int64_t G = C >> 3;
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const int64_t row = row0 + r < R ? row0 + r : R - 1;  // clamped rows are never stored
            w[r] = reinterpret_cast<const uint4 *>(w_base + row * C);
            s[r] = signs + row * G;
            a[r] = PER_MATRIX ? alpha[0] : alpha[row];
        }
    }
};

// ---------------------------------------------------------------- m <= 4
template <int MT, int RW, int D, bool PER_MATRIX>
__global__ __launch_bounds__(512) void gemv_direct(const uint16_t *__restrict__ x, int m,
                                                   const uint16_t *__restrict__ w_base,
                                                   const uint8_t *__restrict__ signs,
                                                   const float *__restrict__ alpha, int64_t R, int64_t C,
                                                   uint16_t *__restrict__ y)
{
    constexpr int kWaves = 8;
    const int lane = threadIdx.x & 63;
    const int64_t row0 = ((int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6)) * RW;
    const int64_t G = C >> 3;
    const int S = (int)((G + 63) >> 6);  // a multiple of D (host checks)
    const Rows<RW, PER_MATRIX> rows(w_base, signs, alpha, row0, R, C);
    const uint4 *xrow[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
        xrow[t] = reinterpret_cast<const uint4 *>(x) + (int64_t)(t < m ? t : m - 1) * G;

    uint4 wq[D][RW], xq[D][MT];
    uint32_t sq[D][RW];
    auto load = [&](int d, int s) {
        const int64_t g0 = (int64_t)s * 64 + lane;
        const int64_t g = g0 < G ? g0 : G - 1;
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            wq[d][r] = rows.w[r][g];
            sq[d][r] = rows.s[r][g];
        }
#pragma unroll
        for (int t = 0; t < MT; ++t)
            xq[d][t] = xrow[t][g];
    };
    float acc[RW * MT];
#pragma unroll
    for (int i = 0; i < RW * MT; ++i)
        acc[i] = 0.0f;
    auto compute = [&](int d, int s) {
        const bool live = (int64_t)s * 64 + lane < G;  // false only in a ragged last step
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            uint4 e = weff_group(wq[d][r], sq[d][r], rows.a[r]);
            if (!live)
                e = make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                float c = acc[r * MT + t];
                c = dot2(e.x, xq[d][t].x, c);
                c = dot2(e.y, xq[d][t].y, c);
                c = dot2(e.z, xq[d][t].z, c);
                c = dot2(e.w, xq[d][t].w, c);
                acc[r * MT + t] = c;
            }
        }
    };
#pragma unroll
    for (int d = 0; d < D; ++d)
        load(d, d);
    for (int s0 = 0; s0 < S - D; s0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            compute(d, s0 + d);
            load(d, s0 + d + D);
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
        compute(d, S - D + d);
    store_rows<RW, MT>(acc, row0, R, m, y);
}

// ------------------------------------------------------------ m in 5..16
// Activations staged in LDS, SLAB_STEPS steps (of 512 columns) at a time.
template <int MT, int RW, int D, bool PER_MATRIX>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemv_lds(const uint16_t *__restrict__ x, int m,
                                                const uint16_t *__restrict__ w_base,
                                                const uint8_t *__restrict__ signs,
                                                const float *__restrict__ alpha, int64_t R, int64_t C,
                                                uint16_t *__restrict__ y)
{
    constexpr int kWaves = 4;
    constexpr int kThreads = 64 * kWaves;
    constexpr int SLAB_STEPS = kMaxLdsBytes / (16 * 64 * MT);  // 8 for MT = 16
    extern __shared__ uint4 xs[];                               // [MT][SLAB_STEPS * 64]
    const int lane = threadIdx.x & 63;
    const int64_t row0 = ((int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6)) * RW;
    const int64_t G = C >> 3;
    const int S = (int)((G + 63) >> 6);
    const Rows<RW, PER_MATRIX> rows(w_base, signs, alpha, row0, R, C);
    const uint4 *x4 = reinterpret_cast<const uint4 *>(x);

    uint4 wq[D][RW];
    uint32_t sq[D][RW];
    auto load = [&](int d, int s) {
        const int64_t g0 = (int64_t)s * 64 + lane;
        const int64_t g = g0 < G ? g0 : G - 1;
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            wq[d][r] = rows.w[r][g];
            sq[d][r] = rows.s[r][g];
        }
    };
    float acc[RW * MT];
#pragma unroll
    for (int i = 0; i < RW * MT; ++i)
        acc[i] = 0.0f;
    auto compute = [&](int d, int s, int s_base) {
        const bool live = (int64_t)s * 64 + lane < G;
        uint4 e[RW];
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            e[r] = weff_group(wq[d][r], sq[d][r], rows.a[r]);
            if (!live)
                e[r] = make_uint4(0, 0, 0, 0);
        }
        const int lg = (s - s_base) * 64 + lane;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const uint4 xv = xs[t * (SLAB_STEPS * 64) + lg];
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                float c = acc[r * MT + t];
                c = dot2(e[r].x, xv.x, c);
                c = dot2(e[r].y, xv.y, c);
                c = dot2(e[r].z, xv.z, c);
                c = dot2(e[r].w, xv.w, c);
                acc[r * MT + t] = c;
            }
        }
    };

    for (int base = 0; base < S; base += SLAB_STEPS) {
        const int n = min(SLAB_STEPS, S - base);  // steps in this slab, a multiple of D
        __syncthreads();
        // Direct-to-LDS loads, 1 KB per wave instruction, all in flight at
        // once.  Sources are clamped into x: tokens >= m read token m-1 and
        // columns past the row read its last group, so every staged value is
        // finite (their products are discarded or multiplied by zero).
        for (int q = threadIdx.x >> 6; q < MT * SLAB_STEPS; q += kWaves) {
            const int t = q / SLAB_STEPS, c = q - t * SLAB_STEPS;
            const int64_t g0 = (int64_t)(base + c) * 64 + lane;
            const int64_t g = g0 < G ? g0 : G - 1;
            const uint4 *src = x4 + (int64_t)(t < m ? t : m - 1) * G + g;
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1))) *)src,
                (void __attribute__((address_space(3))) *)(xs + t * (SLAB_STEPS * 64) + c * 64), 16, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0): the staged slab has landed
        __syncthreads();
#pragma unroll
        for (int d = 0; d < D; ++d)
            load(d, base + d);
        for (int s0 = base; s0 < base + n - D; s0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                compute(d, s0 + d, base);
                load(d, s0 + d + D);
            }
        }
#pragma unroll
        for (int d = 0; d < D; ++d)
            compute(d, base + n - D + d, base);
    }
    store_rows<RW, MT>(acc, row0, R, m, y);
}

int pipeline_depth(int64_t S, int dmax)
{
    int d = dmax;
    while (d > 1 && S % d != 0)
        --d;
    return d;
}

template <int MT, int RW, int D>
hipError_t launch_direct(const uint16_t *x, int m, const uint16_t *w_base, const uint8_t *signs,
                         const float *alpha, bool per_matrix, int64_t d_out, int64_t d_in, uint16_t *y,
                         hipStream_t s)
{
    const int64_t rows_per_block = 8 * RW;
    const dim3 grid((unsigned)((d_out + rows_per_block - 1) / rows_per_block)), block(512);
    if (per_matrix)
        hipLaunchKernelGGL((gemv_direct<MT, RW, D, true>), grid, block, 0, s, x, m, w_base, signs, alpha, d_out, d_in, y);
    else
        hipLaunchKernelGGL((gemv_direct<MT, RW, D, false>), grid, block, 0, s, x, m, w_base, signs, alpha, d_out, d_in, y);
    return hipGetLastError();
}

template <int MT, int RW, int D>
hipError_t launch_lds(const uint16_t *x, int m, const uint16_t *w_base, const uint8_t *signs,
                      const float *alpha, bool per_matrix, int64_t d_out, int64_t d_in, uint16_t *y,
                      hipStream_t s)
{
    const int64_t rows_per_block = 4 * RW;
    const dim3 grid((unsigned)((d_out + rows_per_block - 1) / rows_per_block)), block(256);
    constexpr int lds = kMaxLdsBytes;
    // LDS above the 64 KB default must be requested once per kernel.
    static const bool lds_ok = [] {
        return hipFuncSetAttribute(reinterpret_cast<const void *>(&gemv_lds<MT, RW, D, true>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, lds) == hipSuccess &&
               hipFuncSetAttribute(reinterpret_cast<const void *>(&gemv_lds<MT, RW, D, false>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, lds) == hipSuccess;
    }();
    if (!lds_ok)
        return hipErrorInvalidConfiguration;
    if (per_matrix)
        hipLaunchKernelGGL((gemv_lds<MT, RW, D, true>), grid, block, lds, s, x, m, w_base, signs, alpha, d_out, d_in, y);
    else
        hipLaunchKernelGGL((gemv_lds<MT, RW, D, false>), grid, block, lds, s, x, m, w_base, signs, alpha, d_out, d_in, y);
    return hipGetLastError();
}

// D must divide the number of 512-column steps; pick the largest allowed.
template <int MT, int RW>
hipError_t dispatch_direct(const uint16_t *x, int m, const uint16_t *w, const uint8_t *sg, const float *a, bool pm,
                           int64_t d_out, int64_t d_in, uint16_t *y, hipStream_t s, int dmax)
{
    const int64_t S = ((d_in >> 3) + 63) >> 6;
    switch (pipeline_depth(S, dmax)) {
    case 8: if constexpr (MT == 1) return launch_direct<MT, RW, 8>(x, m, w, sg, a, pm, d_out, d_in, y, s);
            [[fallthrough]];
    case 7: if constexpr (MT == 1) return launch_direct<MT, RW, 7>(x, m, w, sg, a, pm, d_out, d_in, y, s);
            [[fallthrough]];
    case 6: if constexpr (MT == 1) return launch_direct<MT, RW, 6>(x, m, w, sg, a, pm, d_out, d_in, y, s);
            [[fallthrough]];
    case 5: if constexpr (MT == 1) return launch_direct<MT, RW, 5>(x, m, w, sg, a, pm, d_out, d_in, y, s);
            [[fallthrough]];
    case 4: return launch_direct<MT, RW, 4>(x, m, w, sg, a, pm, d_out, d_in, y, s);
    case 3: return launch_direct<MT, RW, 3>(x, m, w, sg, a, pm, d_out, d_in, y, s);
    case 2: return launch_direct<MT, RW, 2>(x, m, w, sg, a, pm, d_out, d_in, y, s);
    default: return launch_direct<MT, RW, 1>(x, m, w, sg, a, pm, d_out, d_in, y, s);
    }
}

// For the LDS kernels D must divide every slab's step count: the full slab
// (a power of two) and the last one.
template <int MT, int RW>
hipError_t dispatch_lds(const uint16_t *x, int m, const uint16_t *w, const uint8_t *sg, const float *a, bool pm,
                        int64_t d_out, int64_t d_in, uint16_t *y, hipStream_t s)
{
    constexpr int slab = kMaxLdsBytes / (16 * 64 * MT);
    const int64_t S = ((d_in >> 3) + 63) >> 6;
    const int64_t last = S % slab == 0 ? std::min<int64_t>(S, slab) : S % slab;
    int d = 4;
    while (d > 1 && (last % d != 0 || (S > slab && slab % d != 0)))
        --d;
    switch (d) {
    case 4: return launch_lds<MT, RW, 4>(x, m, w, sg, a, pm, d_out, d_in, y, s);
    case 3: return launch_lds<MT, RW, 3>(x, m, w, sg, a, pm, d_out, d_in, y, s);
    case 2: return launch_lds<MT, RW, 2>(x, m, w, sg, a, pm, d_out, d_in, y, s);
    default: return launch_lds<MT, RW, 1>(x, m, w, sg, a, pm, d_out, d_in, y, s);
    }
}

}  // namespace

hipError_t launch_gemv(const uint16_t *x, int m, const uint16_t *w_base, const uint8_t *signs,
                       const float *alpha, bool per_matrix, int64_t d_out, int64_t d_in,
                       uint16_t *y, hipStream_t s)
{
    if (m <= 1)
        return dispatch_direct<1, 2>(x, m, w_base, signs, alpha, per_matrix, d_out, d_in, y, s, 8);
    if (m <= 2)
        return dispatch_direct<2, 2>(x, m, w_base, signs, alpha, per_matrix, d_out, d_in, y, s, 4);
    if (m <= 4)
        return dispatch_direct<4, 2>(x, m, w_base, signs, alpha, per_matrix, d_out, d_in, y, s, 4);
    if (m <= 8)
        return dispatch_lds<8, 4>(x, m, w_base, signs, alpha, per_matrix, d_out, d_in, y, s);
    return dispatch_lds<16, 4>(x, m, w_base, signs, alpha, per_matrix, d_out, d_in, y, s);
}

}  // namespace bd

// K-Merge similarity over the full task vectors Delta = W_ft - W_base.
//
// "BitDelta: Serving 14 Zen Models from One GPU Cluster", section "K-Merge:
// Online LoRA Adapter Management for the Edge": step 1 of the pool policy
// compares adapters by the cosine similarity of their task vectors; section
// "MonoSoup" defines a checkpoint's task vector as its weights minus the
// base weights.  Here, for V fine-tuned copies W_ft of one matrix,
// Delta_v = fl32(W_ft_v - f32(W_base)) and the output is the Gram matrix
// <Delta_a, Delta_b> with the cosines it implies (the form over the stored
// 1-bit code is in similarity.hip).
//
// Fixed fp64 order (the same bits on every call and GPU): the product of two
// fp32 values is exact in fp64, so one fma per product rounds exactly as an
// add of the exact product would.  Row term of row r and pair a <= b: 64
// partial sums, 8-column group g into partial g mod 64 (its columns in
// increasing order, groups in increasing g), then the halving tree
// p[k] += p[k + s], s = 32 .. 1.  Row terms: row r into partial r mod 256 in
// increasing r, then the halving tree s = 128 .. 1.
//
// Two kernels.
//  simdelta_rows<NT>: one workgroup per row, one wave per block of a 4 x 4
//    tile pair of variants (NT tiles of 4 variants; NT (NT + 1) / 2 waves).
//    Per 512-column step the workgroup stages Delta of every variant for the
//    step into LDS once (each W_ft byte and each W_base byte read once from
//    HBM, streamed, every load instruction 1 KB contiguous), double-buffered,
//    the loads of step s + 1 in flight while step s is consumed; lane l of
//    every wave owns group 64 s + l of the step, which is exactly partial l
//    of the fixed order, and keeps the fp64 partials of its block's pairs (a
//    diagonal block only those with i <= j; the blocks are ordered so that
//    the SIMDs carry near-equal shares).  The lane halving tree then runs by
//    shuffles and lane 0 writes each pair's row term (fp64 [pairs][R], the
//    caller's workspace).
//  simdelta_gram: one workgroup per pair a <= b sums the row terms of
//    (a, b), (a, a) and (b, b) in the row order above and forms the cosine.
//
// HBM-bound: (4 B per weight per variant for fp32 W_ft, 2 B for bf16) + 2 B
// per weight of W_base; 2 flop per weight and pair of fp64 arithmetic.
#include <hip/hip_runtime.h>

#include "bd_device.h"
#include "bd_launch.h"

namespace bd {
namespace {

constexpr int kSdTile = 4;          // variants per tile
constexpr int kSdTree = 256;        // threads of the Gram kernel

__host__ __device__ constexpr int sd_waves(int nt) { return nt * (nt + 1) / 2; }

// Packed index of pair a <= b: row a of the upper triangle, diagonal included.
__host__ __device__ constexpr int sd_pair(int a, int b, int V) { return a * V - a * (a - 1) / 2 + (b - a); }

// Tile pair (ti, tj), ti <= tj, of wave w.  The waves of a workgroup are
// spread over the CU's 4 SIMDs in turn (wave w on SIMD w mod 4), and a
// diagonal block forms 10 products per column against 16 for the others, so
// at NT = 4 (10 waves) the order puts one off-diagonal and two diagonal
// blocks on each of the SIMDs that hold three waves: 36, 36, 32, 32 products
// per column against 48, 48, 32, 32 in row order.  Otherwise, row order.
template <int NT>
__device__ __forceinline__ void sd_block(int w, int &ti, int &tj)
{
    if constexpr (NT == 4) {
        constexpr int8_t kI[10] = {0, 0, 0, 1, 0, 1, 1, 2, 2, 3};
        constexpr int8_t kJ[10] = {1, 2, 3, 2, 0, 1, 3, 3, 2, 3};
        ti = kI[w];
        tj = kJ[w];
    } else {
        int i = 0, idx = w;
        while (idx >= NT - i) {
            idx -= NT - i;
            ++i;
        }
        ti = i;
        tj = i + idx;
    }
}

template <int NT, bool FT_F32>
__global__ __launch_bounds__(64 * sd_waves(NT)) void simdelta_rows(const uint16_t *__restrict__ w_base,
                                                                   const void *__restrict__ w_ft, int V, int64_t R,
                                                                   int64_t C, double *__restrict__ terms)
{
    constexpr int NW = sd_waves(NT);
    constexpr int NV = NT * kSdTile;                    // variant slots (those >= V hold zeros)
    constexpr int ITEMS = (NV + NW - 1) / NW;           // (variant, group) items staged per thread and step
    // Delta of one step: [buffer][variant][half][lane], 16 bytes = 4 columns;
    // lane l's 8 columns are half 0 and half 1 of its entry (each read is a
    // contiguous 1 KB across the wave: no bank conflict)
    __shared__ uint4 dl[2][NV][2][64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t r = blockIdx.x;
    const int64_t G = C >> 3;
    const int S = (int)((G + 63) >> 6);
    const uint16_t *brow = w_base + r * C;

    // block of this wave: tile pair (ti, tj), ti <= tj
    int ti, tj;
    sd_block<NT>(wave, ti, tj);
    const bool diag = ti == tj;   // a diagonal block forms only its i <= j products

    // staging item k of this thread: variant slot v = (tid + k 64 NW) / 64 and
    // lane gl = tid % 64 (the same for every k, 64 NW being a multiple of 64).
    // bf16 W_ft: lane gl loads the 8 columns of group 64 s + gl (16 bytes of
    // W_ft and of W_base: each load instruction 1 KB contiguous).  fp32 W_ft:
    // lane gl loads columns 512 s + 4 gl .. + 3 and 512 s + 256 + 4 gl .. + 3
    // (two 16-byte loads, each instruction again 1 KB contiguous; W_base by
    // two 8-byte loads), which are the halves gl % 2 of groups 64 s + gl / 2
    // and 64 s + 32 + gl / 2 in LDS.
    const int gl = (int)threadIdx.x & 63;
    struct Raw {
        uint4 f[FT_F32 ? 2 : 1];
        uint4 b;   // W_base: bf16 -> 8 columns; fp32 -> x, y = quarter 0, z, w = quarter 1
    };
    Raw raw[ITEMS];
    auto load = [&](int s) {
        if constexpr (FT_F32) {
            const int64_t c0 = (int64_t)s * 512 + 4 * gl, c1 = c0 + 256;
            const bool ok0 = c0 < C, ok1 = c1 < C;
            const uint2 b0 = ok0 ? *reinterpret_cast<const uint2 *>(brow + c0) : make_uint2(0, 0);
            const uint2 b1 = ok1 ? *reinterpret_cast<const uint2 *>(brow + c1) : make_uint2(0, 0);
#pragma unroll
            for (int k = 0; k < ITEMS; ++k) {
                const int v = ((int)threadIdx.x + k * 64 * NW) >> 6;
                raw[k].b = make_uint4(b0.x, b0.y, b1.x, b1.y);
                const float *f = static_cast<const float *>(w_ft) + ((int64_t)v * R + r) * C;
                raw[k].f[0] = v < V && ok0 ? ld_stream16(f + c0) : make_uint4(0, 0, 0, 0);
                raw[k].f[1] = v < V && ok1 ? ld_stream16(f + c1) : make_uint4(0, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int k = 0; k < ITEMS; ++k) {
                const int v = ((int)threadIdx.x + k * 64 * NW) >> 6;
                const int64_t g = (int64_t)s * 64 + gl;
                const bool ok = v < V && g < G;
                if (ok) {
                    raw[k].b = *reinterpret_cast<const uint4 *>(brow + 8 * g);
                    raw[k].f[0] = ld_stream16(static_cast<const uint16_t *>(w_ft) + ((int64_t)v * R + r) * C + 8 * g);
                } else {
                    raw[k].b = make_uint4(0, 0, 0, 0);
                    raw[k].f[0] = make_uint4(0, 0, 0, 0);
                }
            }
        }
    };
    // Delta = fl32(W_ft - W_base) of each staged item into LDS (zeros for
    // variant slots past V and columns past the row: zero products, which
    // leave a partial unchanged)
    auto store = [&](int buf) {
#pragma unroll
        for (int k = 0; k < ITEMS; ++k) {
            const int v = ((int)threadIdx.x + k * 64 * NW) >> 6;
            if (v >= NV)
                continue;
            const uint4 b = raw[k].b;
            const float base[8] = {lo_f32(b.x), hi_f32(b.x), lo_f32(b.y), hi_f32(b.y),
                                   lo_f32(b.z), hi_f32(b.z), lo_f32(b.w), hi_f32(b.w)};
            float ft[8];
            if constexpr (FT_F32) {
                const uint4 a0 = raw[k].f[0], a1 = raw[k].f[1];
                ft[0] = __uint_as_float(a0.x); ft[1] = __uint_as_float(a0.y);
                ft[2] = __uint_as_float(a0.z); ft[3] = __uint_as_float(a0.w);
                ft[4] = __uint_as_float(a1.x); ft[5] = __uint_as_float(a1.y);
                ft[6] = __uint_as_float(a1.z); ft[7] = __uint_as_float(a1.w);
            } else {
                const uint4 f = raw[k].f[0];
                ft[0] = lo_f32(f.x); ft[1] = hi_f32(f.x); ft[2] = lo_f32(f.y); ft[3] = hi_f32(f.y);
                ft[4] = lo_f32(f.z); ft[5] = hi_f32(f.z); ft[6] = lo_f32(f.w); ft[7] = hi_f32(f.w);
            }
            float d[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                d[i] = ft[i] - base[i];
            const uint4 q0 = make_uint4(__float_as_uint(d[0]), __float_as_uint(d[1]), __float_as_uint(d[2]),
                                        __float_as_uint(d[3]));
            const uint4 q1 = make_uint4(__float_as_uint(d[4]), __float_as_uint(d[5]), __float_as_uint(d[6]),
                                        __float_as_uint(d[7]));
            if constexpr (FT_F32) {
                dl[buf][v][gl & 1][gl >> 1] = q0;
                dl[buf][v][gl & 1][32 + (gl >> 1)] = q1;
            } else {
                dl[buf][v][0][gl] = q0;
                dl[buf][v][1][gl] = q1;
            }
        }
    };

    double acc[kSdTile][kSdTile];
#pragma unroll
    for (int i = 0; i < kSdTile; ++i)
#pragma unroll
        for (int j = 0; j < kSdTile; ++j)
            acc[i][j] = 0.0;

    // this lane's group 64 s + lane of the step in LDS buffer buf, columns in
    // increasing order, half by half
    auto compute = [&](int buf) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint4 qa[kSdTile], qb[kSdTile];
#pragma unroll
            for (int i = 0; i < kSdTile; ++i)
                qa[i] = dl[buf][ti * kSdTile + i][h][lane];
            if (!diag) {
#pragma unroll
                for (int i = 0; i < kSdTile; ++i)
                    qb[i] = dl[buf][tj * kSdTile + i][h][lane];
            }
            if (diag) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    double da[kSdTile];
#pragma unroll
                    for (int i = 0; i < kSdTile; ++i)
                        da[i] = (double)__uint_as_float(c == 0 ? qa[i].x : c == 1 ? qa[i].y : c == 2 ? qa[i].z : qa[i].w);
#pragma unroll
                    for (int i = 0; i < kSdTile; ++i)
#pragma unroll
                        for (int j = i; j < kSdTile; ++j)
                            acc[i][j] = __builtin_fma(da[i], da[j], acc[i][j]);
                }
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    double da[kSdTile], db[kSdTile];
#pragma unroll
                    for (int i = 0; i < kSdTile; ++i) {
                        const uint32_t ua = c == 0 ? qa[i].x : c == 1 ? qa[i].y : c == 2 ? qa[i].z : qa[i].w;
                        const uint32_t ub = c == 0 ? qb[i].x : c == 1 ? qb[i].y : c == 2 ? qb[i].z : qb[i].w;
                        da[i] = (double)__uint_as_float(ua);
                        db[i] = (double)__uint_as_float(ub);
                    }
#pragma unroll
                    for (int i = 0; i < kSdTile; ++i)
#pragma unroll
                        for (int j = 0; j < kSdTile; ++j)
                            acc[i][j] = __builtin_fma(da[i], db[j], acc[i][j]);
                }
            }
        }
    };

    load(0);
    for (int s = 0; s < S; ++s) {
        const int buf = s & 1;
        store(buf);
        __syncthreads();
        if (s + 1 < S)
            load(s + 1);
        compute(buf);
        // the next store writes the other buffer, last read in step s - 1,
        // which every wave finished before this step's barrier
    }

    // halving tree over the 64 lane partials (lane k < s adds lane k + s)
#pragma unroll
    for (int i = 0; i < kSdTile; ++i)
#pragma unroll
        for (int j = 0; j < kSdTile; ++j) {
            double v = acc[i][j];
#pragma unroll
            for (int s = 32; s >= 1; s >>= 1)
                v = v + __shfl_down(v, s, 64);
            acc[i][j] = v;
        }
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < kSdTile; ++i)
#pragma unroll
            for (int j = 0; j < kSdTile; ++j) {
                const int a = ti * kSdTile + i, b = tj * kSdTile + j;
                if (a < V && b < V && a <= b)
                    terms[(int64_t)sd_pair(a, b, V) * R + r] = acc[i][j];
            }
    }
}

// Gram kernel: workgroup (a, b), a <= b, sums the row terms of (a, b),
// (a, a) and (b, b): thread t adds rows t, t + 256, ... in increasing order
// (one batch's loads issued before its adds), then the halving tree in LDS.
constexpr int kSdBatch = 16;

__global__ __launch_bounds__(kSdTree) void simdelta_gram(const double *__restrict__ terms, int V, int64_t R,
                                                        double *__restrict__ gram, double *__restrict__ cosine)
{
    __shared__ double tree[3][kSdTree];
    int a = 0, idx = (int)blockIdx.x;
    while (idx >= V - a) {
        idx -= V - a;
        ++a;
    }
    const int b = a + idx;
    const int t = threadIdx.x;
    const double *tab = terms + (int64_t)sd_pair(a, b, V) * R;
    const double *taa = terms + (int64_t)sd_pair(a, a, V) * R;
    const double *tbb = terms + (int64_t)sd_pair(b, b, V) * R;
    double sab = 0.0, saa = 0.0, sbb = 0.0;
    for (int64_t r0 = t; r0 < R; r0 += (int64_t)kSdBatch * kSdTree) {
        double vab[kSdBatch], vaa[kSdBatch], vbb[kSdBatch];
#pragma unroll
        for (int u = 0; u < kSdBatch; ++u) {
            const int64_t rr = r0 + (int64_t)u * kSdTree;
            const bool ok = rr < R;
            const int64_t ri = ok ? rr : R - 1;
            vab[u] = ok ? tab[ri] : 0.0;
            vaa[u] = ok ? taa[ri] : 0.0;
            vbb[u] = ok ? tbb[ri] : 0.0;
        }
        // a row past R adds +0 to a partial that is never -0: no change
#pragma unroll
        for (int u = 0; u < kSdBatch; ++u) {
            sab = sab + vab[u];
            saa = saa + vaa[u];
            sbb = sbb + vbb[u];
        }
    }
    tree[0][t] = sab;
    tree[1][t] = saa;
    tree[2][t] = sbb;
    __syncthreads();
    for (int s = kSdTree / 2; s >= 1; s >>= 1) {
        if (t < s) {
#pragma unroll
            for (int i = 0; i < 3; ++i)
                tree[i][t] = tree[i][t] + tree[i][t + s];
        }
        __syncthreads();
    }
    if (t == 0) {
        const double gab = tree[0][0], gaa = tree[1][0], gbb = tree[2][0];
        const double n = sqrt(gaa * gbb);
        const double cs = n > 0.0 ? gab / n : 0.0;
        gram[a * V + b] = gab;
        gram[b * V + a] = gab;
        cosine[a * V + b] = cs;
        cosine[b * V + a] = cs;
    }
}

template <int NT>
hipError_t launch_rows(const uint16_t *w_base, const void *w_ft, bool ft_f32, int V, int64_t R, int64_t C,
                       double *terms, hipStream_t s)
{
    const dim3 grid((unsigned)R), block(64 * sd_waves(NT));
    if (ft_f32)
        hipLaunchKernelGGL((simdelta_rows<NT, true>), grid, block, 0, s, w_base, w_ft, V, R, C, terms);
    else
        hipLaunchKernelGGL((simdelta_rows<NT, false>), grid, block, 0, s, w_base, w_ft, V, R, C, terms);
    return hipGetLastError();
}

}  // namespace

size_t similarity_delta_workspace_bytes(int32_t n_variants, int64_t d_out)
{
    if (n_variants < 1 || d_out <= 0)
        return 0;
    return sizeof(double) * (size_t)d_out * (size_t)(n_variants * (n_variants + 1) / 2);
}

hipError_t launch_similarity_delta(const uint16_t *w_base, const void *w_ft, bool ft_f32, int32_t n_variants,
                                   int64_t d_out, int64_t d_in, double *gram, double *cosine, double *terms,
                                   hipStream_t s)
{
    const int nt = (n_variants + kSdTile - 1) / kSdTile;
    hipError_t e;
    switch (nt) {
    case 1: e = launch_rows<1>(w_base, w_ft, ft_f32, n_variants, d_out, d_in, terms, s); break;
    case 2: e = launch_rows<2>(w_base, w_ft, ft_f32, n_variants, d_out, d_in, terms, s); break;
    case 3: e = launch_rows<3>(w_base, w_ft, ft_f32, n_variants, d_out, d_in, terms, s); break;
    case 4: e = launch_rows<4>(w_base, w_ft, ft_f32, n_variants, d_out, d_in, terms, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess)
        return e;
    const int pairs = n_variants * (n_variants + 1) / 2;
    hipLaunchKernelGGL(simdelta_gram, dim3((unsigned)pairs), dim3(kSdTree), 0, s, terms, (int)n_variants, d_out,
                       gram, cosine);
    return hipGetLastError();
}

}  // namespace bd

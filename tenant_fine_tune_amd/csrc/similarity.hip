// Similarity of task vectors for K-Merge-style adapter pooling.
//
// "BitDelta: Serving 14 Zen Models from One GPU Cluster", section "K-Merge:
// Online LoRA Adapter Management for the Edge": step 1 of the pool policy
// compares a newly requested adapter with every pooled one by the cosine
// similarity of their task vectors.  Here a variant's task vector is the
// delta a BitDelta server holds for one matrix, tau[r][j] = alpha[r] * s[r][j]
// (s = +1 for bit 1, -1 for bit 0; section "Mathematical Foundation"), and
// the output is the Gram matrix <tau_a, tau_b> of all variants with the
// cosines it implies.
//
// Two kernels.
//  similarity_counts<V>: the integer part.  For a row r and a pair a < b,
//    c_ab[r] = sum_j s_a s_b = d_in - 2 popcount(signs_a[r] XOR signs_b[r]):
//    exact, so it may be summed in any order.  A workgroup of 4 waves takes
//    16 rows; lane (j, q) = (l % 16, l / 16) of wave w reads, for every
//    variant, the 16 bytes q of the 64-byte chunks k = w, w + 4, ... of row
//    j (the 4 lanes of a row read 64 contiguous bytes per instruction), and
//    keeps one disagreement count per pair (v_xor + v_bcnt per dword and
//    pair).  The counts of the 4 lanes of a row are summed by lane shuffles,
//    those of the 4 waves through LDS, and c_ab[r] is stored as int32
//    [pairs][d_out].  The traffic is the packed signs (d_in / 8 bytes per row
//    and variant); at 14 variants the 91 pairs' v_bcnt work costs about as
//    much as the reads.
//  similarity_gram: the floating-point part, in the fixed order the oracle
//    defines.  One workgroup per pair a <= b: thread t adds, for rows
//    r = t, t + 256, ... in increasing order, the term
//    (alpha_a[r] * alpha_b[r]) * c_ab[r] (the first product is exact in fp64,
//    the second rounds once; no fused multiply-add) into its partial, then
//    the halving tree p[k] += p[k + s], s = 128 .. 1.  The workgroup forms
//    the two diagonal sums alongside, the same way, so the cosine
//    g_ab / sqrt(g_aa g_bb) needs no second launch.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "bd_device.h"
#include "bd_launch.h"

namespace bd {
namespace {

constexpr int kSimWaves = 4;
constexpr int kSimRows = 16;  // rows per workgroup
constexpr int kTreeThreads = 256;

// Pair index of a < b in the packed upper triangle, row by row.
__host__ __device__ constexpr int pair_index(int a, int b, int V) { return a * V - a * (a + 1) / 2 + (b - a - 1); }

// EVEN: d_in / 8 is a multiple of 64 (whole 64-byte chunks); otherwise the
// bytes past the row in the last chunk read as zero in every variant, so
// they add no disagreement.
template <int V, bool EVEN>
__global__ __launch_bounds__(64 * kSimWaves) void similarity_counts(const uint8_t *__restrict__ signs, int64_t R,
                                                                    int64_t C, int32_t *__restrict__ counts)
{
    constexpr int P = V * (V - 1) / 2;
    __shared__ int32_t part[kSimWaves][kSimRows][P];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 15, q = lane >> 4;
    const int64_t G = C >> 3;  // sign bytes per row
    const int64_t row = (int64_t)blockIdx.x * kSimRows + j;
    const bool row_ok = row < R;
    const int nk = (int)((G + 63) >> 6);  // 64-byte chunks per row
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(signs, (int64_t)V * R * G);
    // variant v's row: v * R * G + row * G; lane piece: + 16 q (+ 64 k)
    const uint32_t base = row_ok ? (uint32_t)(row * G + 16 * q) : kInvalidOffset;
    const uint32_t vstride = (uint32_t)(R * G);

    uint32_t d[P];
#pragma unroll
    for (int p = 0; p < P; ++p)
        d[p] = 0;
    // Chunk k of this lane's row for every variant.  The scalar offset (the
    // chunk's position and the variant's block) is outside the hardware range
    // check, so it only moves inside valid rows: with whole chunks (EVEN) a
    // chunk k < nk lies inside the row, and chunks past it (k >= nk) use the
    // out-of-range lane offset (zeros: no disagreement).  With a ragged last
    // chunk each dword gets its own lane offset (d_in % 32 == 0 makes the row
    // a whole number of dwords), out of range past the row: zeros in every
    // variant, so they add no disagreement either.
    auto load = [&](uint4 (&s)[V], int k) {
        if constexpr (EVEN) {
            const uint32_t b = k < nk ? base : kInvalidOffset;
            const uint32_t off = (uint32_t)k * 64u;
#pragma unroll
            for (int v = 0; v < V; ++v)
                s[v] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     rs, b, off + (uint32_t)v * vstride, kStream));
        } else {
            const int64_t start = (int64_t)k * 64 + 16 * q;
            uint32_t vo[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                vo[i] = (row_ok && start + 4 * i < G) ? base + (uint32_t)(k * 64 + 4 * i) : kInvalidOffset;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                s[v].x = __builtin_amdgcn_raw_buffer_load_b32(rs, vo[0], (uint32_t)v * vstride, kStream);
                s[v].y = __builtin_amdgcn_raw_buffer_load_b32(rs, vo[1], (uint32_t)v * vstride, kStream);
                s[v].z = __builtin_amdgcn_raw_buffer_load_b32(rs, vo[2], (uint32_t)v * vstride, kStream);
                s[v].w = __builtin_amdgcn_raw_buffer_load_b32(rs, vo[3], (uint32_t)v * vstride, kStream);
            }
        }
    };
    auto count = [&](uint4 (&s)[V], int k) {
        (void)k;
#pragma unroll
        for (int a = 0; a < V; ++a)
#pragma unroll
            for (int b = a + 1; b < V; ++b) {
                uint32_t c = d[pair_index(a, b, V)];
                c += __builtin_popcount(s[a].x ^ s[b].x);
                c += __builtin_popcount(s[a].y ^ s[b].y);
                c += __builtin_popcount(s[a].z ^ s[b].z);
                c += __builtin_popcount(s[a].w ^ s[b].w);
                d[pair_index(a, b, V)] = c;
            }
    };
    for (int k = wave; k < nk; k += kSimWaves) {
        uint4 s[V];
        load(s, k);
        count(s, k);
    }
    // the 4 lanes of a row (q = 0..3: lanes j, j + 16, j + 32, j + 48)
#pragma unroll
    for (int p = 0; p < P; ++p) {
        uint32_t c = d[p];
        c += __shfl_xor(c, 16, 64);
        c += __shfl_xor(c, 32, 64);
        d[p] = c;
    }
#pragma unroll
    for (int p = 0; p < P; ++p)
        if ((p & 3) == q)
            part[wave][j][p] = (int32_t)d[p];
    __syncthreads();
    // c_ab[r] = d_in - 2 * (disagreements summed over the 4 waves), stored
    // pair-major [pairs][d_out] so the fixed-order sum reads it contiguously
    for (int i = threadIdx.x; i < kSimRows * P; i += 64 * kSimWaves) {
        const int p = i / kSimRows, rr = i - p * kSimRows;
        const int64_t r = (int64_t)blockIdx.x * kSimRows + rr;
        if (r >= R)
            continue;
        int64_t dis = 0;
#pragma unroll
        for (int w = 0; w < kSimWaves; ++w)
            dis += part[w][rr][p];
        counts[(int64_t)p * R + r] = (int32_t)(C - 2 * dis);
    }
}

// The Gram kernel: workgroup (a, b), a <= b, forms g_ab, g_aa and g_bb
// together.  Each is the fixed-order fp64 sum over rows of
// (alpha_x[r] alpha_y[r]) c_xy[r] (c = d_in on the diagonal): thread t adds
// rows t, t + 256, ... in increasing order (all of one batch's loads go out
// before its dependent adds), then the halving tree over the 256 partials.
// Every product and sum rounds on its own (no fused multiply-add: the
// compiler would otherwise contract s + p * c into one fma).
constexpr int kGramBatch = 32;

__global__ __launch_bounds__(kTreeThreads) void similarity_gram(const float *__restrict__ alpha, bool per_matrix,
                                                                const int32_t *__restrict__ counts, int V,
                                                                int64_t R, int64_t C, double *__restrict__ gram,
                                                                double *__restrict__ cosine)
{
#pragma clang fp contract(off)
    __shared__ double tree[3][kTreeThreads];
    // workgroup -> pair a <= b, row by row of the upper triangle
    int a = 0, idx = (int)blockIdx.x;
    while (idx >= V - a) {
        idx -= V - a;
        ++a;
    }
    const int b = a + idx;
    const int t = threadIdx.x;
    const float *aa = per_matrix ? alpha + a : alpha + (int64_t)a * R;
    const float *ab = per_matrix ? alpha + b : alpha + (int64_t)b * R;
    const bool diag = a == b;
    // counts through a buffer resource: the diagonal (and one variant, no
    // pairs at all) reads nothing (out-of-range offset)
    const int P = V * (V - 1) / 2;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(counts, (int64_t)P * R * 4);
    const uint32_t cbase = diag ? kInvalidOffset : (uint32_t)((int64_t)pair_index(a, b, V) * R * 4);
    const double cd = (double)C;
    double sab = 0.0, saa = 0.0, sbb = 0.0;
    for (int64_t r0 = t; r0 < R; r0 += (int64_t)kGramBatch * kTreeThreads) {
        // every load unconditional (rows past R read row R - 1 and are then
        // zeroed), so they all go out before the adds
        float fa[kGramBatch], fb[kGramBatch];
        int32_t c[kGramBatch];
#pragma unroll
        for (int u = 0; u < kGramBatch; ++u) {
            const int64_t r = r0 + (int64_t)u * kTreeThreads;
            const bool ok = r < R;
            const int64_t rr = ok ? r : R - 1;
            const float va = aa[per_matrix ? 0 : rr], vb = ab[per_matrix ? 0 : rr];
            const int32_t vc = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rc, cbase + (uint32_t)(rr * 4), 0, 0);
            fa[u] = ok ? va : 0.0f;
            fb[u] = ok ? vb : 0.0f;
            c[u] = ok ? vc : 0;
        }
        // a zeroed row adds +0 (or -0) to a sum that starts at +0: no change
#pragma unroll
        for (int u = 0; u < kGramBatch; ++u) {
            const double da = (double)fa[u], db = (double)fb[u];
            sab = sab + (da * db) * (diag ? cd : (double)c[u]);
            saa = saa + (da * da) * cd;
            sbb = sbb + (db * db) * cd;
        }
    }
    tree[0][t] = sab;
    tree[1][t] = saa;
    tree[2][t] = sbb;
    __syncthreads();
    for (int s = kTreeThreads / 2; s >= 1; s >>= 1) {
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

template <int V>
hipError_t launch_counts(const uint8_t *signs, int64_t R, int64_t C, int32_t *counts, hipStream_t s)
{
    const dim3 grid((unsigned)((R + kSimRows - 1) / kSimRows)), block(64 * kSimWaves);
    if ((C >> 3) % 64 == 0)
        hipLaunchKernelGGL((similarity_counts<V, true>), grid, block, 0, s, signs, R, C, counts);
    else
        hipLaunchKernelGGL((similarity_counts<V, false>), grid, block, 0, s, signs, R, C, counts);
    return hipGetLastError();
}

template <int V>
hipError_t dispatch_counts(int v, const uint8_t *signs, int64_t R, int64_t C, int32_t *counts, hipStream_t s)
{
    if constexpr (V > kSimilarityMaxVariants)
        return hipErrorInvalidValue;
    else if (v == V)
        return launch_counts<V>(signs, R, C, counts, s);
    else
        return dispatch_counts<V + 1>(v, signs, R, C, counts, s);
}

}  // namespace

size_t similarity_workspace_bytes(int32_t n_variants, int64_t d_out)
{
    if (n_variants < 2 || d_out <= 0)
        return 0;
    return sizeof(int32_t) * (size_t)d_out * (size_t)(n_variants * (n_variants - 1) / 2);
}

hipError_t launch_similarity(const uint8_t *signs, const float *alpha, bool per_matrix, int32_t n_variants,
                             int64_t d_out, int64_t d_in, double *gram, double *cosine, int32_t *counts,
                             hipStream_t s)
{
    if (n_variants >= 2) {
        const hipError_t e = dispatch_counts<2>(n_variants, signs, d_out, d_in, counts, s);
        if (e != hipSuccess)
            return e;
    }
    const int pairs = n_variants * (n_variants + 1) / 2;
    hipLaunchKernelGGL(similarity_gram, dim3((unsigned)pairs), dim3(kTreeThreads), 0, s, alpha, per_matrix, counts,
                       (int)n_variants, d_out, d_in, gram, cosine);
    return hipGetLastError();
}

}  // namespace bd

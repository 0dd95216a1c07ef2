// Prefill kernel: fused BitDelta linear on bf16 MFMA, and its grouped form.
//
// "BitDelta: Serving 14 Zen Models from One GPU Cluster", section "Serving
// Architecture": reconstruction and the matrix product are fused in one
// kernel pass, the effective weight existing only in registers / on-chip
// memory (the conceptual fused_bitdelta_linear sketch fixes the semantics
// y = x (W_base + alpha * unpack(signs))^T); the diagram's delta cache puts
// many variants over one shared, HBM-resident W_base, which the grouped form
// serves in one launch.
//
// Tile: 256 tokens x 256 output features per workgroup, K stepped by 64.
// Four waves; wave w owns output features [64w, 64w+64) of the tile for all
// 256 tokens (8 x 2 blocks of v_mfma_f32_32x32x16_bf16, 256 fp32
// accumulators per lane).  Per K step:
//  - the 256 x 64 activation tile is staged in LDS (rows padded by 16 bytes
//    so the 16-byte fragment reads of 32 consecutive rows hit distinct banks);
//  - each wave loads its own 64 x 64 slice of W_base directly in the MFMA
//    B-operand layout (lane l: feature l%32, 8 consecutive k) plus the sign
//    bytes, forms W_eff = bf16(W_base + +-alpha) in VGPRs and feeds it to the
//    MFMA without any LDS round trip: each weight is rebuilt exactly once per
//    workgroup;
//  - the next step's global loads are issued before the MFMAs of this one.
// Workgroups are remapped so that the ones sharing an output-feature tile run
// on the same XCD (blocks are dealt round-robin over the 8 XCDs), so each
// W_base tile is fetched into one L2 once.
#include "bd_device.h"
#include "bd_launch.h"

namespace bd {
namespace {

constexpr int BM = kGemmBM, BN = kGemmBN, BK = 64;
constexpr int LDS_LD = BK + 8;  // bf16 per LDS row
constexpr int kThreads = 256;
constexpr int kXcds = 8;

__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t nb)
{
    const int64_t per = nb / kXcds;
    if (b >= per * kXcds)
        return b;
    return (b % kXcds) * per + b / kXcds;
}

struct Stage {
    uint4 xr[8];
    uint4 wr[2][4];
    uint32_t sr[2][4];
};

// GATHER = false: tile rows are tokens m0 .. m0+255 of x.
// GATHER = true : tile rows are the tokens listed in rows_s (grouped path).
template <bool PER_MATRIX, bool GATHER>
__device__ __forceinline__ void load_stage(Stage &st, const uint16_t *__restrict__ x, int64_t M,
                                           const int32_t *rows_s, int64_t m0,
                                           const uint16_t *__restrict__ w_base,
                                           const uint8_t *__restrict__ signs, int64_t N, int64_t K,
                                           int64_t n_lane0, int64_t k0, int lane)
{
    const int64_t G = K >> 3;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int q = threadIdx.x + kThreads * i;
        const int row = q >> 3, c = q & 7;
        const int64_t kc = k0 + c * 8;
        int64_t tok;
        if constexpr (GATHER)
            tok = rows_s[row];
        else
            tok = m0 + row < M ? m0 + row : -1;
        st.xr[i] = (tok >= 0 && kc < K) ? *reinterpret_cast<const uint4 *>(x + tok * K + kc)
                                         : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int64_t n = n_lane0 + nb * 32;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int64_t kc = k0 + kb * 16 + 8 * (lane >> 5);
            const bool ok = n < N && kc < K;
            st.wr[nb][kb] = ok ? *reinterpret_cast<const uint4 *>(w_base + n * K + kc) : make_uint4(0, 0, 0, 0);
            st.sr[nb][kb] = ok ? (uint32_t)signs[n * G + (kc >> 3)] : 0u;
        }
    }
}

template <bool PER_MATRIX, bool GATHER>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_tiles(const uint16_t *__restrict__ x, int64_t M, const uint16_t *__restrict__ w_base,
                const uint8_t *__restrict__ signs_all, const float *__restrict__ alpha_all,
                int64_t N, int64_t K, uint16_t *__restrict__ y, int64_t m_tiles,
                const int32_t *__restrict__ table, int32_t n_variants)
{
    __shared__ __attribute__((aligned(16))) uint16_t xs[BM * LDS_LD];
    __shared__ int32_t rows_s[BM];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t b = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t mt = b % m_tiles, nt = b / m_tiles;
    const int64_t n0 = nt * BN;

    int64_t m0 = mt * BM;
    const uint8_t *signs = signs_all;
    const float *alpha = alpha_all;
    if constexpr (GATHER) {
        // table: [0] total tiles, then perm[M], tile_v[T], tile_row0[T], tile_rows[T]
        const int32_t total = table[0];
        if (mt >= total)
            return;
        const int32_t *perm = table + 4;
        const int32_t *tile_v = perm + M;
        const int32_t *tile_row0 = tile_v + m_tiles;
        const int32_t *tile_rows = tile_row0 + m_tiles;
        const int v = tile_v[mt];
        const int row0 = tile_row0[mt], nrows = tile_rows[mt];
        for (int i = threadIdx.x; i < BM; i += kThreads)
            rows_s[i] = i < nrows ? perm[row0 + i] : -1;
        __syncthreads();
        if (v >= n_variants) {
            // tokens whose variant id is out of range: zero rows
            for (int i = 0; i < nrows; ++i) {
                const int64_t tok = rows_s[i];
                for (int64_t j = n0 + threadIdx.x; j < min(N, n0 + BN); j += kThreads)
                    y[tok * N + j] = 0;
            }
            return;
        }
        signs = signs_all + (int64_t)v * N * (K >> 3);
        alpha = PER_MATRIX ? alpha_all + v : alpha_all + (int64_t)v * N;
        m0 = 0;
    }

    const int64_t n_lane0 = n0 + wave * 64 + (lane & 31);
    float a[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int64_t n = n_lane0 + nb * 32;
        a[nb] = PER_MATRIX ? alpha[0] : (n < N ? alpha[n] : 0.0f);
    }

    f32x16 acc[8][2];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[mb][nb][v] = 0.0f;

    Stage st;
    load_stage<PER_MATRIX, GATHER>(st, x, M, rows_s, m0, w_base, signs, N, K, n_lane0, 0, lane);

    for (int64_t k0 = 0; k0 < K; k0 += BK) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int q = threadIdx.x + kThreads * i;
            *reinterpret_cast<uint4 *>(&xs[(q >> 3) * LDS_LD + (q & 7) * 8]) = st.xr[i];
        }
        bf16x8 B[2][4];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                B[nb][kb] = __builtin_bit_cast(bf16x8, weff_group(st.wr[nb][kb], st.sr[nb][kb] >> (0), a[nb]));
        if (k0 + BK < K)
            load_stage<PER_MATRIX, GATHER>(st, x, M, rows_s, m0, w_base, signs, N, K, n_lane0, k0 + BK, lane);
        __syncthreads();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int mb = 0; mb < 8; ++mb) {
                const bf16x8 A = *reinterpret_cast<const bf16x8 *>(
                    &xs[(mb * 32 + (lane & 31)) * LDS_LD + kb * 16 + 8 * (lane >> 5)]);
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B[nb][kb], acc[mb][nb], 0, 0, 0);
            }
        }
    }

    // Output: lane l holds feature column l%32 of each 32x32 block; register
    // v holds token row 8*(v/4) + 4*(l/32) + v%4 of the block.
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int64_t j = n_lane0 + nb * 32;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int i = mb * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                int64_t tok;
                if constexpr (GATHER)
                    tok = rows_s[i];
                else
                    tok = m0 + i < M ? m0 + i : -1;
                if (tok >= 0 && j < N)
                    y[tok * N + j] = to_bf16(acc[mb][nb][v]);
            }
        }
    }
}

// Bucket tokens by variant id in one workgroup: counts, exclusive scan, a
// scatter into per-variant segments, and the tile table of the grouped GEMM.
// Out-of-range ids form one extra bucket (index n_variants) whose tiles
// write zero rows.  Order inside a segment is not fixed, and need not be:
// every output row is computed on its own, in the same arithmetic order
// wherever its token sits in a tile.
constexpr int kBucketThreads = 1024;
constexpr int kMaxVariants = 4096;

__global__ __launch_bounds__(kBucketThreads) void bucket_tokens(const int32_t *__restrict__ ids, int64_t M,
                                                                int32_t V, int64_t max_tiles,
                                                                int32_t *__restrict__ table)
{
    __shared__ int32_t cnt[kMaxVariants + 1];
    __shared__ int32_t seg[kMaxVariants + 2];
    __shared__ int32_t tstart[kMaxVariants + 2];
    const int nb = V + 1;
    for (int i = threadIdx.x; i < nb; i += kBucketThreads)
        cnt[i] = 0;
    __syncthreads();
    for (int64_t t = threadIdx.x; t < M; t += kBucketThreads) {
        const int32_t v = ids[t];
        atomicAdd(&cnt[(v >= 0 && v < V) ? v : V], 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t s = 0, ts = 0;
        for (int i = 0; i < nb; ++i) {
            seg[i] = s;
            tstart[i] = ts;
            s += cnt[i];
            ts += (cnt[i] + BM - 1) / BM;
        }
        seg[nb] = s;
        tstart[nb] = ts;
        table[0] = ts;
        table[1] = table[2] = table[3] = 0;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nb; i += kBucketThreads)
        cnt[i] = seg[i];  // reuse as scatter cursors
    __syncthreads();
    int32_t *perm = table + 4;
    for (int64_t t = threadIdx.x; t < M; t += kBucketThreads) {
        const int32_t v = ids[t];
        const int bkt = (v >= 0 && v < V) ? v : V;
        perm[atomicAdd(&cnt[bkt], 1)] = (int32_t)t;
    }
    int32_t *tile_v = perm + M;
    int32_t *tile_row0 = tile_v + max_tiles;
    int32_t *tile_rows = tile_row0 + max_tiles;
    const int32_t total = tstart[nb];
    for (int ti = threadIdx.x; ti < total; ti += kBucketThreads) {
        int lo = 0, hi = nb - 1;  // last bucket with tstart <= ti
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tstart[mid] <= ti)
                lo = mid;
            else
                hi = mid - 1;
        }
        // skip empty buckets that share the same start
        while (lo + 1 < nb && tstart[lo + 1] <= ti)
            ++lo;
        const int32_t r0 = seg[lo] + (ti - tstart[lo]) * BM;
        tile_v[ti] = lo;
        tile_row0[ti] = r0;
        tile_rows[ti] = min(BM, seg[lo + 1] - r0);
    }
}

template <bool GATHER>
hipError_t launch_tiles(const uint16_t *x, int64_t m, const uint16_t *w_base, const uint8_t *signs,
                        const float *alpha, bool per_matrix, int64_t d_out, int64_t d_in, uint16_t *y,
                        int64_t m_tiles, const int32_t *table, int32_t n_variants, hipStream_t s)
{
    const int64_t n_tiles = (d_out + BN - 1) / BN;
    const dim3 grid((unsigned)(m_tiles * n_tiles)), block(kThreads);
    if (per_matrix)
        hipLaunchKernelGGL((gemm_tiles<true, GATHER>), grid, block, 0, s, x, m, w_base, signs, alpha, d_out, d_in, y,
                           m_tiles, table, n_variants);
    else
        hipLaunchKernelGGL((gemm_tiles<false, GATHER>), grid, block, 0, s, x, m, w_base, signs, alpha, d_out, d_in, y,
                           m_tiles, table, n_variants);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint16_t *x, int64_t m, const uint16_t *w_base, const uint8_t *signs,
                       const float *alpha, bool per_matrix, int64_t d_out, int64_t d_in,
                       uint16_t *y, hipStream_t s)
{
    const int64_t m_tiles = (m + BM - 1) / BM;
    return launch_tiles<false>(x, m, w_base, signs, alpha, per_matrix, d_out, d_in, y, m_tiles, nullptr, 0, s);
}

int64_t grouped_max_tiles(int64_t m, int32_t n_variants)
{
    return (m + BM - 1) / BM + (int64_t)n_variants + 1;
}

size_t grouped_workspace_bytes(int64_t m, int32_t n_variants)
{
    return sizeof(int32_t) * (size_t)(4 + m + 3 * grouped_max_tiles(m, n_variants));
}

hipError_t launch_grouped(const uint16_t *x, int64_t m, const int32_t *ids, int32_t n_variants,
                          const uint16_t *w_base, const uint8_t *signs, const float *alpha,
                          bool per_matrix, int64_t d_out, int64_t d_in, uint16_t *y,
                          int32_t *workspace, hipStream_t s)
{
    const int64_t T = grouped_max_tiles(m, n_variants);
    hipLaunchKernelGGL(bucket_tokens, dim3(1), dim3(kBucketThreads), 0, s, ids, m, n_variants, T, workspace);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    return launch_tiles<true>(x, m, w_base, signs, alpha, per_matrix, d_out, d_in, y, T, workspace, n_variants, s);
}

}  // namespace bd

// MonoSoup merge of k fine-tuned checkpoints on gfx950.
//
// "BitDelta: Serving 14 Zen Models from One GPU Cluster", section "MonoSoup":
// each checkpoint's task vector Delta_i = W_i - W_base is cut to its rank-r
// truncated SVD tau_i, and W_merged = W_base + (1/k) sum_i tau_i.  Delta_i is
// the fp32 difference fl32(W_i - f32(W_base)), formed on the fly from the
// checkpoint and the bf16 base wherever it is read; it is never stored.
//
// The truncation is found by a randomized range finder (Halko, Martinsson and
// Tropp, "Finding structure with randomness", SIAM Review 2011, algorithms
// 4.3/4.4 and 5.1) with a sketch of kMsL = 64 columns and the caller's
// Gaussian test matrix Omega [C, 64]:
//   Y = Delta Omega;  q times: Y <- Y T_Y, Z = Delta^T Y, Z <- Z T_Z,
//   Y = Delta Z;  then Z = Delta^T Y  (T_X: whitening factor of X^T X, below).
// With T the pivoted-Cholesky whitening factor of G = Y^T Y (T^T G T = I on
// the numerical range of Y, directions below 1e-12 of the largest squared
// column norm dropped), Q = Y T has orthonormal columns and
// B = Q^T Delta = T^T Z^T, so B B^T = T^T (Z^T Z) T = U diag(mu) U^T.  The
// rank-r truncation of Q B is Q U_r U_r^T B = (Y P)(Z P)^T with P = T U_r,
// and sqrt(mu) are the estimated singular values.  The merge is then one
// contraction over k * rp columns (rp = r rounded up to 16):
//   W_merged = f32(W_base) + [Y_1 P_1 / k, ...] [Z_1 P_1, ...]^T.
//
// Kernels (every checkpoint in one launch, grid.z or grid.y = checkpoint):
//   ms_pass<TRANS>  Delta (or Delta^T) times a [*, 64] fp32 matrix, split over
//                   the contraction into partials; 64x64 output tile per
//                   workgroup, four waves of v_mfma_f32_32x32x2_f32, the Delta
//                   and right tiles staged through LDS, next tile's global
//                   loads in flight during the MFMAs.  6 bytes (fp32 W_i,
//                   bf16 W_base) and 2 * 64 flop per weight: 21 flop/B, at
//                   the fp32-MFMA ridge (157.3 TFLOP/s over 8 TB/s).
//   ms_reduce       sums the partials in split order (deterministic).
//   ms_gram         fp64 X^T X of a [n, 64] fp32 matrix, at most 256 partials
//                   of consecutive rows (fp32 products are exact in fp64);
//                   ms_gram_reduce sums the partials in a fixed order.
//   ms_whiten       one workgroup of 512: the pivoted-Cholesky whitening
//                   factor T of a 64 x 64 Gram matrix (fp64; one wave factors
//                   with the rows in registers, then 8 lanes per column invert
//                   the triangle).
//   ms_solve        one workgroup of 512: T of Y's Gram, T^T H T, its
//                   eigenvectors by one-sided Jacobi (fp64, columns held in
//                   registers, 2 per group of 16 lanes, a ring ordering that
//                   moves one column per pair and round) and P = T U_r.
//   ms_apply        X T for a [n, 64] matrix and a 64 x ncols fp64 factor,
//                   fp64 accumulation, fp32 result into a strided destination.
//   ms_merge        f32(W_base) + U W^T, 64x64 tiles, v_mfma_f32_32x32x2_f32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bd_device.h"
#include "bd_launch.h"

namespace bd {

namespace {

constexpr int kL = kMsL;          // sketch width
constexpr int kTile = 64;         // rows / columns of a Delta tile
constexpr int kGramRows = 128;    // rows per LDS batch of the Gram kernel
constexpr int kGramMaxChunks = 256;   // partial Grams per matrix at most
constexpr int kPitch = 65;        // padded LDS row (floats or doubles)
// Delta-pass workgroups to aim for by splitting the contraction: 256 CUs x the
// 4 that fit on one (33 KB of LDS, 112 registers), so a pass is one round of
// long splits (8192 x 8192, k = 2: 2048 workgroups of 16 steps took 3% longer
// per merge than 1024 of 32).
constexpr int kTargetGroups = 1024;
constexpr int kMaxSplits = 32;
constexpr int kJacobiSweeps = 30;

typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16_t mfma_f32(float a, float b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Delta passes.  TRANS = false: out[R, 64] = Delta[R, C] rhs[C, 64].
// TRANS = true: out[C, 64] = Delta^T rhs[R, 64].  grid = (output blocks of 64,
// splits, checkpoints); split s covers contraction steps [s*sps, (s+1)*sps).
// part layout: [checkpoint][split][n_out][64] fp32.
template <bool TRANS>
__global__ __launch_bounds__(256) void ms_pass(const uint16_t *__restrict__ wb, const float *__restrict__ wft,
                                               const float *__restrict__ rhs, int64_t rhs_ck_stride, int64_t R,
                                               int64_t C, int64_t sps, float *__restrict__ part)
{
    __shared__ float D[kTile][kPitch];
    __shared__ __attribute__((aligned(16))) float Rs[kTile][kL];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 31, lk = lane >> 5, wi = wave >> 1, wj = wave & 1;
    const int64_t ck = blockIdx.z, S = gridDim.y, s = blockIdx.y;
    const int64_t n_out = TRANS ? C : R, n_k = TRANS ? R : C;
    const int64_t o0 = (int64_t)blockIdx.x * kTile;
    const int64_t steps = (n_k + kTile - 1) / kTile;
    const int64_t st0 = s * sps, st1 = st0 + sps < steps ? st0 + sps : steps;
    const float *wf_ck = wft + ck * R * C;
    const float *rhs_ck = rhs + ck * rhs_ck_stride;
    const int rr0 = tid >> 4, cc = (tid & 15) * 4;

    f32x4 wf[4], rv[4];
    uint2 wv[4];
    auto load = [&](int64_t step) {
        const int64_t k0 = step * kTile;
        const int64_t tr0 = TRANS ? k0 : o0, tc0 = TRANS ? o0 : k0;
        const int64_t rows = R - tr0 < kTile ? R - tr0 : kTile;
        const auto rf = make_rsrc(wf_ck + tr0 * C, rows * C * 4);
        const auto rb = make_rsrc(wb + tr0 * C, rows * C * 2);
        const int64_t krows = n_k - k0 < kTile ? n_k - k0 : kTile;
        const auto rr = make_rsrc(rhs_ck + k0 * kL, krows * kL * 4);
        const bool col_ok = tc0 + cc < C;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int r = it * 16 + rr0;
            const uint32_t of = col_ok ? (uint32_t)((r * C + tc0 + cc) * 4) : kInvalidOffset;
            const uint32_t ob = col_ok ? (uint32_t)((r * C + tc0 + cc) * 2) : kInvalidOffset;
            wf[it] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rf, of, 0, kStream));
            wv[it] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rb, ob, 0, kStream));
            rv[it] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, (uint32_t)((r * kL + cc) * 4), 0, 0));
        }
    };

    f32x16_t acc;
#pragma unroll
    for (int v = 0; v < 16; ++v)
        acc[v] = 0.0f;

    if (st0 < st1)
        load(st0);
    for (int64_t step = st0; step < st1; ++step) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int r = it * 16 + rr0;
            D[r][cc + 0] = wf[it][0] - lo_f32(wv[it].x);
            D[r][cc + 1] = wf[it][1] - hi_f32(wv[it].x);
            D[r][cc + 2] = wf[it][2] - lo_f32(wv[it].y);
            D[r][cc + 3] = wf[it][3] - hi_f32(wv[it].y);
            *reinterpret_cast<f32x4 *>(&Rs[r][cc]) = rv[it];
        }
        __syncthreads();
        if (step + 1 < st1)
            load(step + 1);
#pragma unroll
        for (int t = 0; t < kTile / 2; ++t) {
            const int k = 2 * t + lk;
            const float a = TRANS ? D[k][32 * wi + li] : D[32 * wi + li][k];
            const float b = Rs[k][32 * wj + li];
            acc = mfma_f32(a, b, acc);
        }
        __syncthreads();
    }

    float *dst = part + ((ck * S + s) * n_out) * kL;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int64_t row = o0 + 32 * wi + 8 * (v >> 2) + 4 * lk + (v & 3);
        if (row < n_out)
            dst[row * kL + 32 * wj + li] = acc[v];
    }
}

// out[ck][n][64] = sum over splits (in order) of part[ck][s][n][64].
__global__ __launch_bounds__(256) void ms_reduce(const float *__restrict__ part, int S, int64_t n,
                                                 float *__restrict__ out)
{
    const int64_t ck = blockIdx.y;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;   // float4 index within a checkpoint
    const int64_t n4 = n * (kL / 4);
    if (e >= n4)
        return;
    const f32x4 *p = reinterpret_cast<const f32x4 *>(part) + ck * S * n4 + e;
    f32x4 s = p[0];
    for (int i = 1; i < S; ++i)
        s += p[i * n4];
    reinterpret_cast<f32x4 *>(out)[ck * n4 + e] = s;
}

// Partial Gram X^T X over rows [blockIdx.x * span, +span) of checkpoint
// blockIdx.y (span a multiple of 128, rows in increasing order, 128 at a time
// through LDS); gpart layout [ck][chunk][64][64] fp64.
__global__ __launch_bounds__(256) void ms_gram(const float *__restrict__ X, int64_t n, int64_t span,
                                               double *__restrict__ gpart)
{
    __shared__ __attribute__((aligned(16))) float xs[kGramRows][kL];
    const int tid = threadIdx.x;
    const int64_t ck = blockIdx.y, c0 = (int64_t)blockIdx.x * span;
    const int64_t c1 = c0 + span < n ? c0 + span : n;
    const float *x = X + ck * n * kL;
    const int a0 = (tid >> 4) * 4, b0 = (tid & 15) * 4;
    double acc[4][4] = {};
    for (int64_t r0 = c0; r0 < c1; r0 += kGramRows) {
#pragma unroll
        for (int it = 0; it < kGramRows * kL / 4 / 256; ++it) {
            const int idx = it * 256 + tid, row = idx >> 4, c4 = (idx & 15) * 4;
            f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
            if (r0 + row < c1)
                v = *reinterpret_cast<const f32x4 *>(x + (r0 + row) * kL + c4);
            *reinterpret_cast<f32x4 *>(&xs[row][c4]) = v;
        }
        __syncthreads();
        for (int r = 0; r < kGramRows; ++r) {
            const f32x4 xa = *reinterpret_cast<const f32x4 *>(&xs[r][a0]);
            const f32x4 xb = *reinterpret_cast<const f32x4 *>(&xs[r][b0]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] += (double)xa[i] * (double)xb[j];
        }
        __syncthreads();
    }
    double *g = gpart + ((ck * gridDim.x + blockIdx.x) * kL) * kL;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            g[(a0 + i) * kL + b0 + j] = acc[i][j];
}

// G[ck] = sum over chunks (in chunk order) of the partial Grams.  Four lanes
// per element each sum every fourth chunk; the four sums are added in a fixed
// order ((s0 + s1) + (s2 + s3)).
__global__ __launch_bounds__(256) void ms_gram_reduce(const double *__restrict__ gpart, int nch,
                                                      double *__restrict__ G)
{
    const int64_t ck = blockIdx.y;
    const int e = blockIdx.x * 64 + (threadIdx.x >> 2), part = threadIdx.x & 3;
    const double *g = gpart + ck * nch * kL * kL + e;
    double s = 0.0;
    for (int c = part; c < nch; c += 4)
        s += g[(int64_t)c * kL * kL];
    const double s1 = __shfl_xor(s, 1);
    const double pair = (part & 1) ? s1 + s : s + s1;      // (s0 + s1) or (s2 + s3), same on both lanes
    const double other = __shfl_xor(pair, 2);
    if (part == 0)
        G[ck * kL * kL + e] = pair + other;
}

// The small solvers run one workgroup of kSolveThreads (8 waves) per
// checkpoint.  They keep their matrices in registers where the algorithm
// allows it; LDS carries only what has to change lanes or waves.
constexpr int kSolveThreads = 512;
// lanes per column in the triangle inversion, rows per thread block in the
// 64 x 64 products, lanes per column pair in the eigensolver
constexpr int kInvLanes = kSolveThreads / 64;
constexpr int kMmRows = 1024 / kSolveThreads;
constexpr int kJacLanes = kSolveThreads / 32;
constexpr int kJacRows = kL / kJacLanes;

// Keeps the compiler from moving memory operations across this point; a
// wave's own LDS instructions execute in issue order, so this orders the
// wave's LDS writes and reads without a workgroup barrier.
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Lane moves within rows of 16 lanes (DPP): quad_perm xor 1 (0xB1), quad_perm
// xor 2 (0x4E), mirror within each half row (0x141), rotate a row by 4 / 8
// lanes (0x124 / 0x128); fp64 moved as two 32-bit halves.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over aligned groups of 4 / 8 lanes; every lane of a group gets the same
// bits (each level adds the same two partial sums in either order).
__device__ __forceinline__ double sum4(double v)
{
    v += dpp_f64<0xB1>(v);
    return v + dpp_f64<0x4E>(v);
}
__device__ __forceinline__ double sum8(double v)
{
    v = sum4(v);
    return v + dpp_f64<0x141>(v);
}
__device__ __forceinline__ double sum16(double v)
{
    v = sum8(v);
    return v + dpp_f64<0x128>(v);
}
template <int N>
__device__ __forceinline__ double sum_lanes(double v)
{
    static_assert(N == 4 || N == 8 || N == 16, "aligned groups of 4, 8 or 16 lanes");
    if constexpr (N == 4)
        return sum4(v);
    else if constexpr (N == 8)
        return sum8(v);
    else
        return sum16(v);
}

__device__ __forceinline__ double lane_f64(double v, int lane)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)b, lane), hi = __builtin_amdgcn_readlane((uint32_t)(b >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Largest value over the wave (fmax, NaN ignored), the same in every lane.
__device__ __forceinline__ double max64(double v)
{
    v = fmax(v, dpp_f64<0xB1>(v));
    v = fmax(v, dpp_f64<0x4E>(v));
    v = fmax(v, dpp_f64<0x124>(v));
    v = fmax(v, dpp_f64<0x128>(v));
    return fmax(fmax(lane_f64(v, 0), lane_f64(v, 16)), fmax(lane_f64(v, 32), lane_f64(v, 48)));
}

__device__ void load_64x64(const double *__restrict__ g, double (*A)[kPitch])
{
    for (int e = threadIdx.x; e < kL * kL; e += kSolveThreads)
        A[e >> 6][e & 63] = g[e];
    __syncthreads();
}

// C = X Y (TX false) or X^T Y (TX true) for 64 x 64 fp64 LDS matrices, each
// sum in increasing order of the contraction index; thread (rg, cg) forms the
// kMmRows x 4 block at rows kMmRows rg, columns 4 cg.  The caller
// synchronises before C is read.
template <bool TX>
__device__ void mm64(const double (*X)[kPitch], const double (*Y)[kPitch], double (*C)[kPitch])
{
    constexpr int RB = kMmRows;
    const int rg = threadIdx.x >> 4, cg = threadIdx.x & 15;
    double acc[RB][4];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = 0.0;
    for (int m = 0; m < kL; ++m) {
        double xv[RB], yv[4];
#pragma unroll
        for (int i = 0; i < RB; ++i)
            xv[i] = TX ? X[m][RB * rg + i] : X[RB * rg + i][m];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            yv[j] = Y[m][4 * cg + j];
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = fma(xv[i], yv[j], acc[i][j]);
    }
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            C[RB * rg + i][4 * cg + j] = acc[i][j];
}

// Whitening factor of a Gram matrix by pivoted Cholesky (the rank-revealing
// form: each step eliminates the largest remaining diagonal; it stops when
// that is at most 1e-12 of the largest initial one, or not positive).  With
// the rho chosen indices perm[0..rho) and G restricted to them = M M^T (M
// lower triangular in pivot order), T[perm[a]][b] = (M^-T)[a][b] for a, b <
// rho and 0 elsewhere, so that T^T G T = I_rho and X T has orthonormal
// columns on the numerical range of X (the rest dropped).
struct CholScratch {
    int perm[kL];
    int rho;
};

// The factorisation, by wave 0 alone: lane i keeps row i of the Schur
// complement in registers and its diagonal entry.  A step picks the largest
// remaining diagonal p (ties to the lower index), forms the pivot column
// l = S[:, p] / sqrt(S[p][p]) (0 in rows already chosen), stores it as
// Lf[:, j] and subtracts l l^T.  Column p is row p (S is symmetric): lane p
// stages its row in `buf`, and l reaches every lane through `buf` too.
// S is only read.
__device__ void pchol_wave(const double (*S)[kPitch], double (*Lf)[kPitch], double *buf, CholScratch &cs)
{
    const int lane = threadIdx.x & 63;
    double s[kL];
#pragma unroll
    for (int m = 0; m < kL; ++m)
        s[m] = S[lane][m];
    double d = S[lane][lane];
    const double dmax0 = max64(d);
    bool chosen = false;
    int rho = 0;
    for (int j = 0; j < kL; ++j) {
        // the largest remaining diagonal, the lowest lane holding it
        const double v = chosen ? -1.0 : d;
        const double dp = max64(v);
        const uint64_t at = __ballot(v == dp);
        if (at == 0 || !(dp > 1e-12 * dmax0) || !(dp > 0.0))
            break;
        const int p = __builtin_ctzll(at);
        const double sd = sqrt(dp);
        if (lane == p) {
#pragma unroll
            for (int m = 0; m < kL; ++m)
                buf[m] = s[m];
        }
        wave_sync();
        const double l = lane == p ? sd : (chosen ? 0.0 : buf[lane] / sd);
        Lf[lane][j] = l;
        if (lane == p) {
            chosen = true;
            cs.perm[j] = p;
        }
        d -= l * l;
        wave_sync();   // every lane has read buf
        buf[lane] = l;
        wave_sync();
#pragma unroll
        for (int m = 0; m < kL; ++m)
            s[m] -= l * buf[m];
        wave_sync();   // before buf is written again
        rho = j + 1;
    }
    if (lane == 0)
        cs.rho = rho;
}

// T from the factorisation (every thread of the workgroup; after a barrier
// that follows pchol_wave): Xi = M^-1 with M[a][m] = Lf[perm[a]][m], by
// forward substitution Xi[a][c] = (delta_ac - sum_{c <= m < a} M[a][m]
// Xi[m][c]) / M[a][a]; column c by the kInvLanes lanes (c, part), lane part
// keeping Xi[m][c] for m = part + kInvLanes k in registers.
// Then T[perm[a]][b] = Xi[b][a] for a, b < rho and 0 elsewhere, written
// through `put(i, j, value)` for every entry.
template <typename Put>
__device__ void whiten_factor(const double (*Lf)[kPitch], const CholScratch &cs, Put put)
{
    constexpr int NL = kInvLanes;
    const int tid = threadIdx.x, c = tid / NL, part = tid % NL;
    const int rho = cs.rho;
    double x[kL / NL];
#pragma unroll
    for (int k = 0; k < kL / NL; ++k)
        x[k] = 0.0;
#pragma unroll
    for (int a = 0; a < kL; ++a) {
        if (a < rho) {
            const int pa = cs.perm[a];
            double s = 0.0;
#pragma unroll
            for (int k = 0; NL * k < a; ++k) {
                const int m = part + NL * k;
                if (m < a && m >= c)
                    s += Lf[pa][m] * x[k];
            }
            s = sum_lanes<NL>(s);
            const double xa = c <= a ? ((c == a ? 1.0 : 0.0) - s) / Lf[pa][a] : 0.0;
            if (part == a % NL)
                x[a / NL] = xa;
        }
    }
    for (int e = tid; e < kL * kL; e += kSolveThreads)
        put(e >> 6, e & 63, 0.0);
    __syncthreads();
    if (c < rho) {
        const int pc = cs.perm[c];
#pragma unroll
        for (int k = 0; k < kL / NL; ++k) {
            const int m = part + NL * k;
            if (m < rho)
                put(pc, m, x[k]);
        }
    }
    __syncthreads();
}

// T (global, [ck][64][64]) = the pivoted-Cholesky whitening factor of G[ck].
__global__ __launch_bounds__(kSolveThreads) void ms_whiten(const double *__restrict__ G, double *__restrict__ T)
{
    __shared__ double S[kL][kPitch];
    __shared__ double Lf[kL][kPitch];
    __shared__ double buf[kL];
    __shared__ CholScratch cs;
    const int64_t ck = blockIdx.x;
    double *t_ck = T + ck * kL * kL;
    load_64x64(G + ck * kL * kL, S);
    if (threadIdx.x < 64)
        pchol_wave(S, Lf, buf, cs);
    __syncthreads();
    whiten_factor(Lf, cs, [&](int i, int j, double v) { t_ck[i * kL + j] = v; });
}

// The rotation (c, s) that zeroes the off-diagonal entry of the symmetric
// 2 x 2 block [[a_pp, a_pq], [a_pq, a_qq]] (its symmetric Schur
// decomposition, Golub and Van Loan, "Matrix Computations": t = s / c the
// root of t^2 + 2 tau t - 1 = 0 of smaller magnitude, tau = (a_qq - a_pp) /
// (2 a_pq)), written with the half angle: with d = a_qq - a_pp, e = 2 a_pq
// and r = sqrt(d^2 + e^2), c^2 = (1 + |d| / r) / 2 and s = sign(d) e / (2 r c)
// (sign(0) = +1).  Two reciprocal square roots, each refined by two Newton
// steps (quadratic: from the instructions' half precision to full fp64), and
// no division; the caller skips a_pq = 0.
__device__ __forceinline__ double2 half_angle_rotation(double app, double aqq, double apq)
{
    const double d = aqq - app, e = 2.0 * apq;
    const double x = fma(d, d, e * e);
    double y = __builtin_amdgcn_rsq(x);
    y = y * fma(-0.5 * x * y, y, 1.5);
    y = y * fma(-0.5 * x * y, y, 1.5);
    const double w = fma(0.5 * fabs(d), y, 0.5);
    double q = __builtin_amdgcn_rsq(w);
    q = q * fma(-0.5 * w * q, q, 1.5);
    q = q * fma(-0.5 * w * q, q, 1.5);
    return make_double2(w * q, (d >= 0.0 ? e : -e) * y * 0.5 * q);
}

// Exchange buffers of the eigensolver: per buffer 32 slots of one column of
// G and one of V (64 rows each) plus 2 doubles of padding.
constexpr int kXSlot = 2 * kL + 2;
constexpr int kXBuf = 32 * kXSlot;   // = kL * kPitch: one [kL][kPitch] array per buffer
static_assert(kXBuf == kL * kPitch, "an exchange buffer fills one 64 x 65 array");

// Eigen-decomposition of the symmetric positive semi-definite M (64 x 64,
// LDS) by one-sided Jacobi (Hestenes): the columns of G = M are rotated in
// pairs, G <- G J and V <- V J, by the rotation that zeroes the pair's inner
// product (the symmetric Schur rotation of the pair's 2 x 2 Gram), until all
// columns are orthogonal.  Then G = M V with orthogonal columns, so V^T M^2 V
// is diagonal: V holds eigenvectors of M, and the column norms of G are its
// eigenvalues (M is positive semi-definite).
//
// Parallel ordering: 32 groups of kJacLanes lanes; a group holds two columns
// (a stationary and a moving slot), each lane keeping kJacRows of the 64 rows
// of both, of G and of V, in registers.  A sweep has phases of 32, 16, 8, 4,
// 2 and 1 rounds.  In a phase with rings of Q groups, each round every group
// rotates its two columns and then hands its moving column to the previous
// group of its ring (cyclically), so every stationary column of a ring meets
// every moving column of it.  Before the next phase, in each block of 2Q
// groups, the lower half's moving columns trade places with the upper half's
// stationary ones and the upper half's moving columns become stationary, so
// that the next phase pairs columns that have not met yet.  Each of the 2016
// pairs meets exactly once per sweep (63 rounds).  Columns change groups
// through LDS (the lanes of a group move contiguous bytes, 16 each, per
// instruction), two buffers used in turn, one workgroup barrier per exchange.
// Stops after a sweep whose largest relative inner product |g_p . g_q| /
// (|g_p| |g_q|) was at most 1e-6 (the quadratic convergence of cyclic Jacobi
// leaves the columns orthogonal to about 1e-12 after that sweep's rotations;
// a threshold of 1e-9 ran one more sweep, 2.5% of a merge at 8192 x 8192),
// or after kJacobiSweeps sweeps.  Output: Vout[:, j] = the eigenvector of
// original column j, mu[j] its eigenvalue.  Every thread of the workgroup
// takes part; Vout may alias M.
__device__ void jacobi_onesided(const double (*M)[kPitch], double *xb, int *xid, int *red,
                                double (*Vout)[kPitch], double *mu)
{
    constexpr int NL = kJacLanes, NR = kJacRows;
    const int tid = threadIdx.x, g = tid / NL, sub = tid % NL;
    // lane `sub` of a group keeps rows 2 sub + 2 NL u + e (e < 2) as entries
    // t = 2 u + e, so that the group's lanes move contiguous bytes of a
    // column per LDS instruction
    auto row = [&](int t) { return 2 * sub + 2 * NL * (t >> 1) + (t & 1); };
    double gs[NR], gm[NR], vs[NR], vm[NR];
    int ids = g, idm = 32 + g;
#pragma unroll
    for (int t = 0; t < NR; ++t) {
        gs[t] = M[row(t)][ids];
        gm[t] = M[row(t)][idm];
        vs[t] = row(t) == ids ? 1.0 : 0.0;
        vm[t] = row(t) == idm ? 1.0 : 0.0;
    }
    int cur = 0;
    auto put = [&](int slot, const double (&gc)[NR], const double (&vc)[NR], int id) {
        double *p = xb + cur * kXBuf + slot * kXSlot;
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            p[row(t)] = gc[t];
            p[kL + row(t)] = vc[t];
        }
        if (sub == 0)
            xid[cur * 32 + slot] = id;
    };
    auto take = [&](int slot, double (&gc)[NR], double (&vc)[NR], int &id) {
        const double *p = xb + cur * kXBuf + slot * kXSlot;
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            gc[t] = p[row(t)];
            vc[t] = p[kL + row(t)];
        }
        id = xid[cur * 32 + slot];
    };
    // the group's two column norms squared and inner product, summed over
    // its lanes (every lane gets the same bits)
    auto gram2 = [&](double &al, double &be, double &ga) {
        al = 0.0;
        be = 0.0;
        ga = 0.0;
#pragma unroll
        for (int t = 0; t < NR; ++t) {
            al = fma(gs[t], gs[t], al);
            be = fma(gm[t], gm[t], be);
            ga = fma(gs[t], gm[t], ga);
        }
        al = sum_lanes<NL>(al);
        be = sum_lanes<NL>(be);
        ga = sum_lanes<NL>(ga);
    };
    for (int sweep = 0; sweep < kJacobiSweeps; ++sweep) {
        bool more = false;  // a pair of this sweep had |g_p . g_q| > 1e-6 |g_p| |g_q|
        for (int Q = 32; Q >= 1; Q >>= 1) {
            if (Q < 32) {
                const bool upper = (g & Q) != 0;
                if (upper)
                    put(g, gs, vs, ids);
                else
                    put(g, gm, vm, idm);
                __syncthreads();
                if (upper) {
#pragma unroll
                    for (int t = 0; t < NR; ++t) {
                        gs[t] = gm[t];
                        vs[t] = vm[t];
                    }
                    ids = idm;
                    take(g - Q, gm, vm, idm);
                } else {
                    take(g + Q, gm, vm, idm);
                }
                cur ^= 1;
            }
            for (int r = 0; r < Q; ++r) {
                double al, be, ga;
                gram2(al, be, ga);
                const double g2 = ga * ga, ab = al * be;
                more |= g2 > 1e-12 * ab;
                if (g2 > 1e-30 * ab) {
                    const double2 cs = half_angle_rotation(al, be, ga);
#pragma unroll
                    for (int t = 0; t < NR; ++t) {
                        const double a = gs[t], b = gm[t];
                        gs[t] = cs.x * a - cs.y * b;
                        gm[t] = cs.y * a + cs.x * b;
                        const double va = vs[t], vb = vm[t];
                        vs[t] = cs.x * va - cs.y * vb;
                        vm[t] = cs.y * va + cs.x * vb;
                    }
                }
                if (Q > 1) {
                    put(g, gm, vm, idm);
                    __syncthreads();
                    take((g & ~(Q - 1)) | ((g + 1) & (Q - 1)), gm, vm, idm);
                    cur ^= 1;
                }
            }
        }
        // any such pair in the workgroup
        const bool wave_more = __ballot(more) != 0;
        if ((tid & 63) == 0)
            red[tid >> 6] = wave_more ? 1 : 0;
        __syncthreads();
        int w = 0;
        for (int i = 0; i < kSolveThreads / 64; ++i)
            w |= red[i];
        if (!w)
            break;
    }
    double al, be, ga;
    gram2(al, be, ga);
    __syncthreads();   // every read of M is done (Vout may alias it)
#pragma unroll
    for (int t = 0; t < NR; ++t) {
        Vout[row(t)][ids] = vs[t];
        Vout[row(t)][idm] = vm[t];
    }
    if (sub == 0) {
        mu[ids] = sqrt(al);
        mu[idm] = sqrt(be);
    }
    __syncthreads();
}

// Per checkpoint: P [64][64] fp64 (columns >= r zero) and sigma[r].
//   T = pivoted-Cholesky whitening of G = Y^T Y (Q = Y T orthonormal on the
//   numerical range of Y); B B^T = T^T H T with H = Z^T Z = U diag(mu) U^T;
//   P = T U_r, sigma = sqrt(mu_r).
__global__ __launch_bounds__(kSolveThreads) void ms_solve(const double *__restrict__ Gy,
                                                          const double *__restrict__ Gz, int r,
                                                          double *__restrict__ P, double *__restrict__ sigma)
{
    __shared__ double A[kL][kPitch];       // Gy, then H, then T^T H T, then its eigenvectors
    __shared__ double Tm[kL][kPitch];      // T
    __shared__ double W2[2][kL][kPitch];   // Lf and H T; the eigensolver's exchange buffers
    __shared__ double buf[kL];
    __shared__ double mu[kL];
    __shared__ int red[kSolveThreads / 64];
    __shared__ int xid[2 * 32];
    __shared__ int order[kL];
    __shared__ CholScratch cs;
    const int tid = threadIdx.x;
    const int64_t ck = blockIdx.x;

    load_64x64(Gy + ck * kL * kL, A);
    if (tid < 64)
        pchol_wave(A, W2[0], buf, cs);
    __syncthreads();
    whiten_factor(W2[0], cs, [&](int i, int j, double v) { Tm[i][j] = v; });

    // A <- H, W2[1] <- H T, A <- T^T (H T), symmetrised
    load_64x64(Gz + ck * kL * kL, A);
    mm64<false>(A, Tm, W2[1]);
    __syncthreads();
    mm64<true>(Tm, W2[1], A);
    __syncthreads();
    for (int e = tid; e < kL * kL; e += kSolveThreads) {
        const int i = e >> 6, j = e & 63;
        if (i < j) {
            const double m = 0.5 * (A[i][j] + A[j][i]);
            A[i][j] = m;
            A[j][i] = m;
        }
    }
    __syncthreads();
    jacobi_onesided(A, &W2[0][0][0], xid, red, A, mu);

    // order the eigenvalues mu decreasing (ties to the lower index)
    if (tid < kL) {
        const double m0 = mu[tid];
        int rank = 0;
        for (int j = 0; j < kL; ++j) {
            const double o = mu[j];
            rank += (o > m0) || (o == m0 && j < tid);
        }
        order[rank] = tid;
    }
    __syncthreads();
    // P = T U_r: thread (rg, cg) forms rows kMmRows rg .., columns 4 cg .. + 3
    double *p_ck = P + ck * kL * kL;
    {
        constexpr int RB = kMmRows;
        const int rg = tid >> 4, cg = tid & 15;
        int oc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            oc[j] = order[4 * cg + j];
        double acc[RB][4];
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = 0.0;
        for (int b = 0; b < kL; ++b) {
            double tv[RB], uv[4];
#pragma unroll
            for (int i = 0; i < RB; ++i)
                tv[i] = Tm[RB * rg + i][b];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                uv[j] = A[b][oc[j]];
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = fma(tv[i], uv[j], acc[i][j]);
        }
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                p_ck[(RB * rg + i) * kL + 4 * cg + j] = 4 * cg + j < r ? acc[i][j] : 0.0;
    }
    if (sigma && tid < r)
        sigma[ck * r + tid] = sqrt(mu[order[tid]]);
}

// dst[ck][row][c] (row stride dst_row, checkpoint stride dst_ck) =
// scale * sum_a X[ck][row][a] F[ck][a][c] for c < ncols; fp64 accumulation.
__global__ __launch_bounds__(256) void ms_apply(const float *__restrict__ X, int64_t n,
                                                const double *__restrict__ F, int ncols, double scale,
                                                float *__restrict__ dst, int64_t dst_row, int64_t dst_ck)
{
    __shared__ double Fs[kL][kL];
    __shared__ float Xs[kTile][kPitch];
    const int tid = threadIdx.x;
    const int64_t ck = blockIdx.y, r0 = (int64_t)blockIdx.x * kTile;
    const double *f = F + ck * kL * kL;
    for (int e = tid; e < kL * kL; e += 256)
        Fs[e >> 6][e & 63] = f[e];
    const float *x = X + ck * n * kL;
    for (int e = tid; e < kTile * kL; e += 256) {
        const int row = e >> 6, a = e & 63;
        Xs[row][a] = r0 + row < n ? x[(r0 + row) * kL + a] : 0.0f;
    }
    __syncthreads();
    // thread (rg, cg): rows 4 rg .. 4 rg + 3, columns 4 cg .. 4 cg + 3 (4 x 4 register block)
    const int rg = tid >> 4, cg = tid & 15;
    double acc[4][4] = {};
    for (int a = 0; a < kL; ++a) {
        double xv[4], fv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xv[i] = Xs[4 * rg + i][a];
            fv[i] = Fs[a][4 * cg + i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] += xv[i] * fv[j];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t row = r0 + 4 * rg + i;
        if (row < n) {
            float *d = dst + ck * dst_ck + row * dst_row;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (4 * cg + j < ncols)
                    d[4 * cg + j] = (float)(acc[i][j] * scale);
        }
    }
}

// out[R, C] = f32(W_base) + U[R, K] W[C, K]^T, K a multiple of 16 (0 allowed).
// The 64 x 64 tile's products (v_mfma_f32_32x32x2_f32, four waves) pass
// through LDS to the epilogue, where 16 lanes cover one tile row: each W_base
// load instruction reads 4 rows x 128 contiguous bytes and each store writes
// 4 rows x 256 contiguous bytes.
constexpr int kMergePitch = 68;   // floats per row of the output tile in LDS (16-byte rows)

__global__ __launch_bounds__(256) void ms_merge(const uint16_t *__restrict__ wb, const float *__restrict__ U,
                                                const float *__restrict__ W, int64_t R, int64_t C, int K,
                                                float *__restrict__ out)
{
    // Us [kk][row] and Ws [kk][col], then the output tile [row][col] over both
    __shared__ __attribute__((aligned(16))) float smem[2 * kTile * kPitch];
    static_assert(2 * kTile * kPitch >= kTile * kMergePitch, "the output tile fits over Us and Ws");
    float(*Us)[kPitch] = reinterpret_cast<float(*)[kPitch]>(smem);
    float(*Ws)[kPitch] = reinterpret_cast<float(*)[kPitch]>(smem + kTile * kPitch);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 31, lk = lane >> 5, wi = wave >> 1, wj = wave & 1;
    const int64_t r0 = (int64_t)blockIdx.y * kTile, c0 = (int64_t)blockIdx.x * kTile;
    const int rr0 = tid >> 4, kq = (tid & 15) * 4;

    // the epilogue's W_base groups (rows rr0 + 16 it, columns kq .. kq + 3),
    // loaded before the MFMAs so they arrive meanwhile
    uint2 bb[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int64_t row = r0 + rr0 + 16 * it, c = c0 + kq;
        bb[it] = (row < R && c < C) ? *reinterpret_cast<const uint2 *>(wb + row * C + c) : make_uint2(0u, 0u);
    }

    f32x16_t acc;
#pragma unroll
    for (int v = 0; v < 16; ++v)
        acc[v] = 0.0f;
    for (int kk0 = 0; kk0 < K; kk0 += kTile) {
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int row = it * 16 + rr0;
            const bool kok = kk0 + kq < K;
            f32x4 u = {0.0f, 0.0f, 0.0f, 0.0f}, w = u;
            if (kok && r0 + row < R)
                u = *reinterpret_cast<const f32x4 *>(U + (r0 + row) * K + kk0 + kq);
            if (kok && c0 + row < C)
                w = *reinterpret_cast<const f32x4 *>(W + (c0 + row) * K + kk0 + kq);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Us[kq + e][row] = u[e];
                Ws[kq + e][row] = w[e];
            }
        }
        __syncthreads();
        const int nk = K - kk0 < kTile ? K - kk0 : kTile;
        for (int t = 0; t < nk / 2; ++t) {
            const int k = 2 * t + lk;
            acc = mfma_f32(Ws[k][32 * wi + li], Us[k][32 * wj + li], acc);
        }
        __syncthreads();
    }
    // acc[v]: column 32 wi + 8 (v / 4) + 4 lk + v % 4, row 32 wj + li of the tile
    float(*T)[kMergePitch] = reinterpret_cast<float(*)[kMergePitch]>(smem);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o[e] = acc[4 * g + e];
        *reinterpret_cast<f32x4 *>(&T[32 * wj + li][32 * wi + 8 * g + 4 * lk]) = o;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int row = rr0 + 16 * it;
        const int64_t gr = r0 + row, gc = c0 + kq;
        if (gr < R && gc < C) {   // C % 4 == 0: the group of four is whole
            const f32x4 p = *reinterpret_cast<const f32x4 *>(&T[row][kq]);
            const uint2 b = bb[it];
            f32x4 o;
            o[0] = lo_f32(b.x) + p[0];
            o[1] = hi_f32(b.x) + p[1];
            o[2] = lo_f32(b.y) + p[2];
            o[3] = hi_f32(b.y) + p[3];
            *reinterpret_cast<f32x4 *>(out + gr * C + gc) = o;
        }
    }
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct PassPlan {
    int64_t sps;   // contraction steps per split
    int S;         // splits
};

PassPlan pass_plan(int64_t n_out, int64_t n_k, int32_t k)
{
    const int64_t blocks = cdiv(n_out, kTile) * k, steps = cdiv(n_k, kTile);
    int64_t want = cdiv(kTargetGroups, blocks);
    want = want < 1 ? 1 : (want > kMaxSplits ? kMaxSplits : want);
    want = want > steps ? steps : want;
    const int64_t sps = cdiv(steps, want);
    return PassPlan{sps, (int)cdiv(steps, sps)};
}

// Rows per partial Gram: a multiple of 128, so that at most 256 partials cover n rows.
int64_t gram_span(int64_t n) { return kGramRows * cdiv(cdiv(n, kGramRows), kGramMaxChunks); }
int gram_chunks(int64_t n) { return (int)cdiv(n, gram_span(n)); }

struct MsLayout {
    size_t part, y, z, x2, gy, gz, g2y, g2z, t, p, u, w, total;
    int nch_y, nch_z, rp, K;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

MsLayout ms_layout(int64_t R, int64_t C, int32_t k, int32_t rank)
{
    MsLayout L{};
    const PassPlan pn = pass_plan(R, C, k), pt = pass_plan(C, R, k);
    const int64_t part_f = (int64_t)k * kL * (pn.S * R > pt.S * C ? pn.S * R : pt.S * C);
    L.nch_y = gram_chunks(R);
    L.nch_z = gram_chunks(C);
    L.rp = (int)cdiv(rank, 16) * 16;
    L.K = k * L.rp;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    L.part = take(part_f * 4);
    L.y = take((size_t)k * R * kL * 4);
    L.z = take((size_t)k * C * kL * 4);
    L.x2 = take((size_t)k * (R > C ? R : C) * kL * 4);
    L.gy = take((size_t)k * L.nch_y * kL * kL * 8);
    L.gz = take((size_t)k * L.nch_z * kL * kL * 8);
    L.g2y = take((size_t)k * kL * kL * 8);
    L.g2z = take((size_t)k * kL * kL * 8);
    L.t = take((size_t)k * kL * kL * 8);
    L.p = take((size_t)k * kL * kL * 8);
    L.u = take((size_t)R * L.K * 4);
    L.w = take((size_t)C * L.K * 4);
    L.total = off;
    return L;
}

}  // namespace

size_t monosoup_workspace_bytes(int64_t R, int64_t C, int32_t k, int32_t rank)
{
    if (rank == 0)
        return 0;
    return ms_layout(R, C, k, rank).total;
}

hipError_t launch_monosoup(const uint16_t *w_base, const float *w_ft, const float *omega, int32_t k, int64_t R,
                           int64_t C, int32_t rank, int32_t power_iters, float *out, double *sigma,
                           void *workspace, hipStream_t s)
{
    const int64_t K = rank == 0 ? 0 : (int64_t)k * cdiv(rank, 16) * 16;
    if (rank == 0) {
        hipLaunchKernelGGL(ms_merge, dim3((unsigned)cdiv(C, kTile), (unsigned)cdiv(R, kTile)), dim3(256), 0, s,
                           w_base, (const float *)nullptr, (const float *)nullptr, R, C, 0, out);
        return hipGetLastError();
    }
    const MsLayout L = ms_layout(R, C, k, rank);
    char *ws = static_cast<char *>(workspace);
    float *part = reinterpret_cast<float *>(ws + L.part);
    float *Y = reinterpret_cast<float *>(ws + L.y);
    float *Z = reinterpret_cast<float *>(ws + L.z);
    float *X2 = reinterpret_cast<float *>(ws + L.x2);
    double *gy = reinterpret_cast<double *>(ws + L.gy);
    double *gz = reinterpret_cast<double *>(ws + L.gz);
    double *G2y = reinterpret_cast<double *>(ws + L.g2y);
    double *G2z = reinterpret_cast<double *>(ws + L.g2z);
    double *T = reinterpret_cast<double *>(ws + L.t);
    double *P = reinterpret_cast<double *>(ws + L.p);
    float *U = reinterpret_cast<float *>(ws + L.u);
    float *W = reinterpret_cast<float *>(ws + L.w);
    const PassPlan pn = pass_plan(R, C, k), pt = pass_plan(C, R, k);

    // out_ = Delta rhs (TRANS false: [R, 64]) or Delta^T rhs (TRANS true: [C, 64])
    auto pass = [&](bool trans, const float *rhs, int64_t rhs_stride, float *o) {
        const PassPlan pp = trans ? pt : pn;
        const int64_t n_out = trans ? C : R;
        const dim3 grid((unsigned)cdiv(n_out, kTile), (unsigned)pp.S, (unsigned)k);
        if (trans)
            hipLaunchKernelGGL(ms_pass<true>, grid, dim3(256), 0, s, w_base, w_ft, rhs, rhs_stride, R, C, pp.sps,
                               part);
        else
            hipLaunchKernelGGL(ms_pass<false>, grid, dim3(256), 0, s, w_base, w_ft, rhs, rhs_stride, R, C, pp.sps,
                               part);
        hipLaunchKernelGGL(ms_reduce, dim3((unsigned)cdiv(n_out * (kL / 4), 256), (unsigned)k), dim3(256), 0, s,
                           part, pp.S, n_out, o);
    };
    // G2 <- X^T X (fp64, per checkpoint)
    auto gram = [&](const float *X, int64_t n, double *g, double *G2) {
        const int nch = gram_chunks(n);
        hipLaunchKernelGGL(ms_gram, dim3((unsigned)nch, (unsigned)k), dim3(256), 0, s, X, n, gram_span(n), g);
        hipLaunchKernelGGL(ms_gram_reduce, dim3(kL * kL / 64, (unsigned)k), dim3(256), 0, s, (const double *)g, nch,
                           G2);
    };
    // X2 <- whiten(X)
    auto whiten = [&](const float *X, int64_t n, double *g, double *G2) {
        gram(X, n, g, G2);
        hipLaunchKernelGGL(ms_whiten, dim3((unsigned)k), dim3(kSolveThreads), 0, s, (const double *)G2, T);
        hipLaunchKernelGGL(ms_apply, dim3((unsigned)cdiv(n, kTile), (unsigned)k), dim3(256), 0, s, X, n,
                           (const double *)T, kL, 1.0, X2, (int64_t)kL, n * kL);
    };

    pass(false, omega, 0, Y);
    for (int it = 0; it < power_iters; ++it) {
        whiten(Y, R, gy, G2y);
        pass(true, X2, R * kL, Z);
        whiten(Z, C, gz, G2z);
        pass(false, X2, C * kL, Y);
    }
    pass(true, Y, R * kL, Z);
    gram(Y, R, gy, G2y);
    gram(Z, C, gz, G2z);
    hipLaunchKernelGGL(ms_solve, dim3((unsigned)k), dim3(kSolveThreads), 0, s, (const double *)G2y,
                       (const double *)G2z, rank, P, sigma);
    hipLaunchKernelGGL(ms_apply, dim3((unsigned)cdiv(R, kTile), (unsigned)k), dim3(256), 0, s, (const float *)Y, R,
                       (const double *)P, L.rp, 1.0 / (double)k, U, K, (int64_t)L.rp);
    hipLaunchKernelGGL(ms_apply, dim3((unsigned)cdiv(C, kTile), (unsigned)k), dim3(256), 0, s, (const float *)Z, C,
                       (const double *)P, L.rp, 1.0, W, K, (int64_t)L.rp);
    hipLaunchKernelGGL(ms_merge, dim3((unsigned)cdiv(C, kTile), (unsigned)cdiv(R, kTile)), dim3(256), 0, s, w_base,
                       (const float *)U, (const float *)W, R, C, (int)K, out);
    return hipGetLastError();
}

}  // namespace bd

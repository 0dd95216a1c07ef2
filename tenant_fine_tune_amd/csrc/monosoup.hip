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
//   ms_whiten       one workgroup of 1024: the pivoted-Cholesky whitening
//                   factor T of a 64 x 64 Gram matrix (fp64).
//   ms_solve        one workgroup of 1024: T of Y's Gram, then a cyclic Jacobi
//                   eigensolve of T^T H T (fp64, 64x64, round-robin parallel
//                   ordering, one 2x2 block update per thread and round) and
//                   P = T U_r.
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
constexpr int kTargetGroups = 2048;
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

// The small solvers run one workgroup of kSolveThreads per checkpoint.
constexpr int kSolveThreads = 1024;
constexpr int kSolveWaves = kSolveThreads / 64;

// Workgroup-wide fp64 sum, fixed order.
__device__ double block_sum(double v, double *red)
{
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o);
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = 0.0;
    for (int w = 0; w < kSolveWaves; ++w)
        s += red[w];
    __syncthreads();
    return s;
}

__device__ void load_64x64(const double *__restrict__ g, double (*A)[kPitch])
{
    for (int e = threadIdx.x; e < kL * kL; e += kSolveThreads)
        A[e >> 6][e & 63] = g[e];
    __syncthreads();
}

// Whitening factor of a Gram matrix by pivoted Cholesky (the rank-revealing
// form: each step eliminates the largest remaining diagonal; it stops when
// that is at most 1e-12 of the largest initial one, or not positive).  With
// the rho chosen indices perm[0..rho) and G restricted to them = M M^T (M
// lower triangular in pivot order), T[perm[a]][b] = (M^-T)[a][b] for a, b <
// rho and 0 elsewhere, so that T^T G T = I_rho and X T has orthonormal
// columns on the numerical range of X (the rest dropped).  S is overwritten
// (Schur complement), Lf receives the pivot columns, Xi is scratch; T is
// written through `put(i, j, value)` for every entry.  Returns rho.
struct CholScratch {
    int perm[kL];
    int chosen[kL];
    double piv_d;
    int piv;
};

template <typename Put>
__device__ int pivoted_whiten(double (*S)[kPitch], double (*Lf)[kPitch], double (*Xi)[kPitch], CholScratch &cs,
                              Put put)
{
    const int tid = threadIdx.x;
    if (tid < kL)
        cs.chosen[tid] = 0;
    double d0 = tid < kL ? S[tid][tid] : 0.0;
    if (tid < 64) {   // wave 0: largest initial diagonal
        for (int o = 32; o > 0; o >>= 1)
            d0 = fmax(d0, __shfl_xor(d0, o));
        if (tid == 0)
            cs.piv_d = d0;
    }
    __syncthreads();
    const double dmax0 = cs.piv_d;
    __syncthreads();
    int rho = 0;
    for (int j = 0; j < kL; ++j) {
        if (tid < 64) {   // wave 0: argmax of the remaining diagonal, ties to the lower index
            double v = cs.chosen[tid] ? -1.0 : S[tid][tid];
            int idx = tid;
            for (int o = 32; o > 0; o >>= 1) {
                const double v2 = __shfl_xor(v, o);
                const int i2 = __shfl_xor(idx, o);
                if (v2 > v || (v2 == v && i2 < idx)) {
                    v = v2;
                    idx = i2;
                }
            }
            if (tid == 0) {
                cs.piv_d = v;
                cs.piv = idx;
            }
        }
        __syncthreads();
        const double dp = cs.piv_d;
        const int p = cs.piv;
        if (!(dp > 1e-12 * dmax0) || !(dp > 0.0))
            break;
        const double sd = sqrt(dp);
        if (tid < kL)
            Lf[tid][j] = tid == p ? sd : (cs.chosen[tid] ? 0.0 : S[tid][p] / sd);
        __syncthreads();
        if (tid == 0) {
            cs.chosen[p] = 1;
            cs.perm[j] = p;
        }
        for (int e = tid; e < kL * kL; e += kSolveThreads) {
            const int i = e >> 6, m = e & 63;
            S[i][m] -= Lf[i][j] * Lf[m][j];
        }
        rho = j + 1;
        __syncthreads();
    }
    // Xi = M^-1 row by row, M[a][b] = Lf[perm[a]][b]: Xi[a][c] = (delta_ac -
    // sum_{c <= m < a} M[a][m] Xi[m][c]) / M[a][a]; 16 lanes per column c
    const int c = tid >> 4, part = tid & 15;
    for (int a = 0; a < rho; ++a) {
        const int pa = cs.perm[a];
        double s = 0.0;
        for (int m = c + part; m < a; m += 16)
            s += Lf[pa][m] * Xi[m][c];
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 4);
        s += __shfl_xor(s, 8);
        if (part == 0)
            Xi[a][c] = c <= a ? ((c == a ? 1.0 : 0.0) - s) / Lf[pa][a] : 0.0;
        __syncthreads();
    }
    // T[perm[a]][b] = Xi[b][a] (a, b < rho); every other entry 0
    for (int e = tid; e < kL * kL; e += kSolveThreads) {
        const int i = e >> 6, b = e & 63;
        put(i, b, 0.0);
    }
    __syncthreads();
    for (int e = tid; e < kL * kL; e += kSolveThreads) {
        const int a = e >> 6, b = e & 63;
        if (a < rho && b < rho)
            put(cs.perm[a], b, Xi[b][a]);
    }
    __syncthreads();
    return rho;
}

// T (global, [ck][64][64]) = the pivoted-Cholesky whitening factor of G[ck].
__global__ __launch_bounds__(kSolveThreads) void ms_whiten(const double *__restrict__ G, double *__restrict__ T)
{
    __shared__ double S[kL][kPitch];
    __shared__ double Lf[kL][kPitch];
    __shared__ double Xi[kL][kPitch];
    __shared__ CholScratch cs;
    const int64_t ck = blockIdx.x;
    double *t_ck = T + ck * kL * kL;
    load_64x64(G + ck * kL * kL, S);
    pivoted_whiten(S, Lf, Xi, cs, [&](int i, int j, double v) { t_ck[i * kL + j] = v; });
}

// Cyclic Jacobi on the symmetric A (64 x 64, LDS); V receives the
// eigenvectors (columns), diag(A) the eigenvalues.  Each sweep visits all
// pairs in 63 rounds of 32 disjoint rotations (round-robin ordering, index
// 63 fixed); the rotation of a pair is the symmetric Schur decomposition of
// its 2 x 2 block (Golub and Van Loan, "Matrix Computations"), with
// t = sign(d) e / (|d| + sqrt(d^2 + e^2)), d = a_qq - a_pp, e = 2 a_pq.
// Within a round, A <- J^T A J is applied as independent 2 x 2 block
// updates, one per thread (row pair x column pair), and V <- V J alongside.
// Stops when the off-diagonal mass is below 1e-22 of the diagonal's.
__device__ __forceinline__ void round_pair(int step, int m, int &p, int &q)
{
    if (m == 0) {
        p = step;
        q = kL - 1;
    } else {
        p = (step + m) % (kL - 1);
        q = (step - m + (kL - 1)) % (kL - 1);
    }
}

// The rotation (c, s) of one pair, t = sign(d) e / (|d| + sqrt(d^2 + e^2)),
// c = 1 / sqrt(1 + t^2), s = t c, from the hardware reciprocal and reciprocal
// square root, each refined by two Newton steps (quadratic: from the
// instructions' half precision to full fp64), so c^2 + s^2 = 1 to rounding.
__device__ __forceinline__ double2 jacobi_rotation(double app, double aqq, double apq)
{
    if (apq == 0.0)
        return make_double2(1.0, 0.0);
    const double d = aqq - app, e = 2.0 * apq;
    const double x = fma(d, d, e * e);
    double y = __builtin_amdgcn_rsq(x);
    y = y * fma(-0.5 * x * y, y, 1.5);
    y = y * fma(-0.5 * x * y, y, 1.5);
    const double den = fabs(d) + x * y;
    double z = __builtin_amdgcn_rcp(den);
    z = z * fma(-den, z, 2.0);
    z = z * fma(-den, z, 2.0);
    const double t = (d >= 0.0 ? e : -e) * z;
    const double u = fma(t, t, 1.0);
    double c = __builtin_amdgcn_rsq(u);
    c = c * fma(-0.5 * u * c, c, 1.5);
    c = c * fma(-0.5 * u * c, c, 1.5);
    return make_double2(c, t * c);
}

__device__ void jacobi_eig(double (*A)[kPitch], double (*V)[kPitch], double2 *rot, double *red)
{
    const int tid = threadIdx.x;
    for (int e = tid; e < kL * kL; e += kSolveThreads)
        V[e >> 6][e & 63] = (e >> 6) == (e & 63) ? 1.0 : 0.0;
    __syncthreads();
    const int m1 = tid >> 5, m2 = tid & 31;          // the block (row pair m1, column pair m2)
    const int vi = tid & 63, vm = tid >> 6;          // V rows: pairs vm and vm + 16
    for (int sweep = 0; sweep < kJacobiSweeps; ++sweep) {
        double off = 0.0, dg = 0.0;
        for (int e = tid; e < kL * kL; e += kSolveThreads) {
            const double a = A[e >> 6][e & 63];
            if ((e >> 6) == (e & 63))
                dg += a * a;
            else
                off += a * a;
        }
        off = block_sum(off, red);
        dg = block_sum(dg, red);
        if (off <= 1e-22 * dg || off == 0.0)
            break;
        for (int step = 0; step < kL - 1; ++step) {
            if (tid < kL / 2) {
                int p, q;
                round_pair(step, tid, p, q);
                rot[tid] = jacobi_rotation(A[p][p], A[q][q], A[p][q]);
            }
            int p1, q1, p2, q2, pa, qa, pb, qb;
            round_pair(step, m1, p1, q1);
            round_pair(step, m2, p2, q2);
            round_pair(step, vm, pa, qa);
            round_pair(step, vm + 16, pb, qb);
            __syncthreads();
            const double2 r1 = rot[m1], r2 = rot[m2], ra = rot[vm], rb = rot[vm + 16];
            const double a = A[p1][p2], b = A[p1][q2], c = A[q1][p2], d = A[q1][q2];
            const double va = V[vi][pa], wa = V[vi][qa], vb = V[vi][pb], wb = V[vi][qb];
            const double rpp = r1.x * a - r1.y * c, rpq = r1.x * b - r1.y * d;   // rows of J1^T X
            const double rqp = r1.y * a + r1.x * c, rqq = r1.y * b + r1.x * d;
            A[p1][p2] = r2.x * rpp - r2.y * rpq;                                // columns of (J1^T X) J2
            A[p1][q2] = r2.y * rpp + r2.x * rpq;
            A[q1][p2] = r2.x * rqp - r2.y * rqq;
            A[q1][q2] = r2.y * rqp + r2.x * rqq;
            V[vi][pa] = ra.x * va - ra.y * wa;
            V[vi][qa] = ra.y * va + ra.x * wa;
            V[vi][pb] = rb.x * vb - rb.y * wb;
            V[vi][qb] = rb.y * vb + rb.x * wb;
            __syncthreads();
        }
    }
}

// Per checkpoint: P [64][64] fp64 (columns >= r zero) and sigma[r].
//   T = pivoted-Cholesky whitening of G = Y^T Y (Q = Y T orthonormal on the
//   numerical range of Y); B B^T = T^T H T with H = Z^T Z = U diag(mu) U^T;
//   P = T U_r, sigma = sqrt(mu_r).
__global__ __launch_bounds__(kSolveThreads) void ms_solve(const double *__restrict__ Gy,
                                                          const double *__restrict__ Gz, int r,
                                                          double *__restrict__ P, double *__restrict__ sigma)
{
    __shared__ double A[kL][kPitch];
    __shared__ double V[kL][kPitch];
    __shared__ double W3[kL][kPitch];
    __shared__ double Tm[kL][kPitch];
    __shared__ CholScratch cs;
    __shared__ double2 rot[kL / 2];
    __shared__ double red[kSolveWaves];
    __shared__ int order[kL];
    const int tid = threadIdx.x;
    const int64_t ck = blockIdx.x;

    load_64x64(Gy + ck * kL * kL, A);
    pivoted_whiten(A, V, W3, cs, [&](int i, int j, double v) { Tm[i][j] = v; });

    // A <- H, V <- H T, A <- T^T (H T), symmetrised
    load_64x64(Gz + ck * kL * kL, A);
    for (int e = tid; e < kL * kL; e += kSolveThreads) {
        const int i = e >> 6, j = e & 63;
        double s = 0.0;
#pragma unroll 4
        for (int m = 0; m < kL; ++m)
            s += A[i][m] * Tm[m][j];
        V[i][j] = s;
    }
    __syncthreads();
    for (int e = tid; e < kL * kL; e += kSolveThreads) {
        const int i = e >> 6, j = e & 63;
        double s = 0.0;
#pragma unroll 4
        for (int m = 0; m < kL; ++m)
            s += Tm[m][i] * V[m][j];
        A[i][j] = s;
    }
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
    jacobi_eig(A, V, rot, red);

    // order the eigenvalues mu decreasing (ties to the lower index)
    if (tid < kL) {
        const double mu = A[tid][tid];
        int rank = 0;
        for (int j = 0; j < kL; ++j) {
            const double o = A[j][j];
            rank += (o > mu) || (o == mu && j < tid);
        }
        order[rank] = tid;
    }
    __syncthreads();
    double *p_ck = P + ck * kL * kL;
    for (int e = tid; e < kL * kL; e += kSolveThreads) {
        const int a = e >> 6, t = e & 63;
        double s = 0.0;
        if (t < r) {
            const int j = order[t];
#pragma unroll 4
            for (int b = 0; b < kL; ++b)
                s += Tm[a][b] * V[b][j];
        }
        p_ck[e] = s;
    }
    if (sigma && tid < r) {
        const double mu = A[order[tid]][order[tid]];
        sigma[ck * r + tid] = sqrt(mu > 0.0 ? mu : 0.0);
    }
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
// The accumulator is computed transposed (A operand = W, B operand = U), so
// each lane holds four consecutive output columns of one row: one 16-byte
// store and one 8-byte W_base load per group of four.
__global__ __launch_bounds__(256) void ms_merge(const uint16_t *__restrict__ wb, const float *__restrict__ U,
                                                const float *__restrict__ W, int64_t R, int64_t C, int K,
                                                float *__restrict__ out)
{
    __shared__ float Us[kTile][kPitch];   // [kk][row]
    __shared__ float Ws[kTile][kPitch];   // [kk][col]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 31, lk = lane >> 5, wi = wave >> 1, wj = wave & 1;
    const int64_t r0 = (int64_t)blockIdx.y * kTile, c0 = (int64_t)blockIdx.x * kTile;
    const int rr0 = tid >> 4, kq = (tid & 15) * 4;

    // the W_base groups of the epilogue, loaded before the MFMAs so they arrive meanwhile
    const int64_t row = r0 + 32 * wj + li;
    uint2 bb[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int64_t c = c0 + 32 * wi + 8 * g + 4 * lk;
        bb[g] = (row < R && c < C) ? *reinterpret_cast<const uint2 *>(wb + row * C + c) : make_uint2(0u, 0u);
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
    // acc[v]: column c0 + 32 wi + 8 (v / 4) + 4 lk + v % 4, row r0 + 32 wj + li
    if (row < R) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int64_t c = c0 + 32 * wi + 8 * g + 4 * lk;
            if (c < C) {   // C % 4 == 0: the group of four is whole
                const uint2 b = bb[g];
                f32x4 o;
                o[0] = lo_f32(b.x) + acc[4 * g + 0];
                o[1] = hi_f32(b.x) + acc[4 * g + 1];
                o[2] = lo_f32(b.y) + acc[4 * g + 2];
                o[3] = hi_f32(b.y) + acc[4 * g + 3];
                *reinterpret_cast<f32x4 *>(out + row * C + c) = o;
            }
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

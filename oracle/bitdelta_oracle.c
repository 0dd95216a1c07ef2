/*
 * BitDelta oracle: plain, slow, obviously correct CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no source, header, table or helper with
 * the GPU library, and it includes nothing from it.
 *
 * Source of the method: "BitDelta: Serving 14 Zen Models from One GPU
 * Cluster" (hanzo.blog, 2026-02-28; the same post in Indonesian, Simplified
 * Chinese and Arabic).  Sections cited below by their English headings:
 *   [MF]  "Mathematical Foundation": the task delta, the 1-bit code
 *         W_ft ~= W_base + alpha * sign(Delta), alpha = (1/n)||Delta||_1.
 *   [SA]  "Serving Architecture": step 3 of the request flow rebuilds
 *         W_eff = W_base + alpha * sign(Delta); the conceptual
 *         fused_bitdelta_linear sketch (unpack to {-1,+1}, add
 *         alpha[:,None] * signs, then a plain linear y = x W_eff^T).
 *   [ID]  "Infrastructure Details": storage format, signs packed 8 per byte
 *         ([4096,4096] -> [4096,512]) and fp32 alpha, one per output row.
 *   [KM]  "K-Merge: Online LoRA Adapter Management for the Edge": step 1 of
 *         its policy compares a new adapter with every pooled one by the
 *         cosine similarity of their task vectors.
 *   [MS]  "MonoSoup" (a single-checkpoint complement by SVD): the task
 *         vectors Delta_i = W_i - W_base of k checkpoints are each cut to
 *         their rank-r truncated SVD tau_i, and W_merged = W_base +
 *         (1/k) sum_i tau_i.
 *
 * Readings where the post is silent (each one is listed in the design notes):
 *   R1 sign(0): Delta >= 0 (including -0) is stored as bit 1 = +1; bit 0 = -1.
 *   R2 bit order: column j of a row is bit (j & 7) of byte (j >> 3).
 *   R3 Delta_ij is the fp32 difference fl32(W_ft - W_base).
 *   R4 alpha: the |Delta| values are summed in fp64 in a fixed order (below),
 *      and the mean is rounded once to fp32, the storage format of [ID].
 *      Per-row mode (one alpha per output row, [ID]) and per-matrix mode
 *      (one scalar, [MF]) are both provided.
 *   R5 W_eff = bf16_rne(fl32(f32(W_base) + (+/-alpha))): the sketch's mixed
 *      dtypes are resolved by adding in fp32 and rounding once to bf16.
 *   R6 linear: y = x W_eff^T accumulated in fp64 (products of two bf16 values
 *      are exact in fp64).  The GPU returns bf16; tests compare against y64.
 *   R7 similarity ([KM]): the task vector of a variant is the delta a BitDelta
 *      server holds, tau[r][j] = alpha[r] * s[r][j] with s = +1 for bit 1 and
 *      -1 for bit 0; the similarity of two variants is the cosine of their
 *      task vectors over one matrix, from the dot products (Gram matrix).
 *   R9 similarity of the full task vectors ([KM] with the task vector of
 *      [MS], Delta = W_ft - W_base): Delta_v = fl32(W_ft_v - f32(W_base)) as
 *      in R3; the Gram matrix <Delta_a, Delta_b> in the fixed fp64 order
 *      given below, cosines as in R7.  R7's form (over the stored 1-bit code)
 *      is kept beside it: a server that holds only the code can use that one.
 *   R8 MonoSoup ([MS]): Delta_i = fl32(W_i - f32(W_base)) as in R3, then
 *      fp64; tau_i = the exact rank-r truncated SVD (the r largest singular
 *      values and their vectors), computed here by one-sided Jacobi in fp64;
 *      W_merged returned in fp64.
 *
 * Fixed order for the Gram matrix (R7).  For variants a, b and row r,
 * c_ab[r] = sum_j s_a[r][j] s_b[r][j] is an integer (exact).  The row term is
 * ((double)alpha_a[r] * (double)alpha_b[r]) * (double)c_ab[r]: the first
 * product is exact in fp64, the second rounds once.  Row terms go into 256
 * fp64 partials, row r into p[r mod 256] in increasing r, then the halving
 * tree below; gram[a][b] = p[0].  cos[a][b] = gram[a][b] /
 * sqrt(gram[a][a] * gram[b][b]) in fp64 (0 when either norm is 0).
 *
 * Fixed order for the full task-vector Gram matrix (R9).  Each product
 * (double)Delta_a[r][j] * (double)Delta_b[r][j] of two fp32 values is exact in
 * fp64 (so a fused multiply-add gives the same result as multiply-then-add).
 * Row term of row r: 64 fp64 partials p[0..63], all +0; the 8-column groups
 * g = 0 .. C/8-1 in increasing order add their eight products, in increasing
 * column order, into p[g mod 64]; then for s = 32, 16, ..., 1: p[k] = p[k] +
 * p[k+s] for k < s; the row term is p[0].  The row terms then follow R7's row
 * order: row r into q[r mod 256] in increasing r, the 256-wide halving tree,
 * gram[a][b] = q[0]; cos[a][b] = gram[a][b] / sqrt(gram[a][a] gram[b][b]) (0
 * when either norm is 0).
 *
 * Fixed summation order for alpha (R4).  For row r with C columns, split the
 * columns into 8-column groups g = 0 .. C/8-1.  There are 256 fp64 partial
 * sums p[0..255], all +0.  Groups are visited in increasing g; group g adds
 * its eight |Delta| values, in increasing column order, into p[g mod 256].
 * Then for s = 128, 64, ..., 1: p[k] = p[k] + p[k+s] for k < s.  S_r = p[0].
 * Per-row:    alpha_r = (float)(S_r / C)                (fp64 divide, one RNE)
 * Per-matrix: q[0..255] = +0; for r increasing, q[r mod 256] += S_r; the same
 *             halving tree; alpha = (float)(q[0] / (R*C)).
 *
 * Parity pins for every function here live in the CPU test tier: hand-built
 * bytes and ties, closed-form means, an exact rational (math.fsum) mean,
 * Laplace statistics, least-squares optimality of alpha, brute-force
 * exact-rational matrix products on tiny inputs, exact rational Gram
 * matrices, and for the MonoSoup merge task vectors with a known SVD,
 * LAPACK's SVD and the Eckart-Young residual.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- bf16 <-> fp32 from the IEEE 754 binary32 layout ------------------- */

/* bf16 is the upper 16 bits of a binary32; widening is exact. */
float oracle_f32_from_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a binary32 to the nearest bf16, ties to even.  NaN becomes the
 * canonical quiet NaN 0x7FC0; Inf stays Inf; overflow rounds to Inf;
 * subnormals are kept (no flush to zero). */
uint16_t oracle_bf16_from_f32(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return 0x7FC0;
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* ---- helpers ------------------------------------------------------------ */

static float w_ft_at(const void *w_ft, int ft_is_f32, int64_t idx)
{
    if (ft_is_f32)
        return ((const float *)w_ft)[idx];
    return oracle_f32_from_bf16(((const uint16_t *)w_ft)[idx]);
}

/* The halving tree over 256 fp64 partial sums used by R4. */
static double halving_tree_256(double *p)
{
    for (int s = 128; s >= 1; s >>= 1)
        for (int k = 0; k < s; ++k)
            p[k] = p[k] + p[k + s];
    return p[0];
}

/* Signed scale for one weight: bit 1 -> +alpha, bit 0 -> -alpha ([SA]
 * sketch: unpack to {-1,+1} then multiply by alpha; the product is exact). */
static float signed_alpha(const uint8_t *sign_row, int64_t j, float a)
{
    int bit = (sign_row[j >> 3] >> (j & 7)) & 1;
    return bit ? a : -a;
}

/* ---- compress: Delta, sign, pack, alpha ([MF], [ID]) -------------------- */

/* w_base: bf16 bits [R, C]; w_ft: fp32 or bf16 [R, C]; signs out [R, C/8];
 * alpha out [R] (per_matrix = 0) or [1] (per_matrix = 1).
 * row_sum_out (may be NULL): the fp64 S_r of every row.
 * Returns 0, or -1 when C is not a multiple of 8 or a size is negative. */
int oracle_compress(const uint16_t *w_base, const void *w_ft, int ft_is_f32,
                    int64_t R, int64_t C, int per_matrix,
                    uint8_t *signs, float *alpha, double *row_sum_out)
{
    if (R < 0 || C <= 0 || C % 8 != 0)
        return -1;
    double *S = (double *)malloc(sizeof(double) * (size_t)(R > 0 ? R : 1));
    if (!S)
        return -2;
    int64_t groups = C / 8;

#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        double p[256];
        for (int k = 0; k < 256; ++k)
            p[k] = 0.0;
        for (int64_t g = 0; g < groups; ++g) {
            uint8_t byte = 0;
            for (int i = 0; i < 8; ++i) {
                int64_t j = 8 * g + i;
                int64_t idx = r * C + j;
                float d = w_ft_at(w_ft, ft_is_f32, idx) - oracle_f32_from_bf16(w_base[idx]);
                if (d >= 0.0f)
                    byte |= (uint8_t)(1u << i);
                p[g % 256] = p[g % 256] + (double)fabsf(d);
            }
            signs[r * groups + g] = byte;
        }
        S[r] = halving_tree_256(p);
    }

    if (!per_matrix) {
        for (int64_t r = 0; r < R; ++r)
            alpha[r] = (float)(S[r] / (double)C);
    } else {
        double q[256];
        for (int k = 0; k < 256; ++k)
            q[k] = 0.0;
        for (int64_t r = 0; r < R; ++r)
            q[r % 256] = q[r % 256] + S[r];
        double T = halving_tree_256(q);
        alpha[0] = (float)(T / ((double)R * (double)C));
    }
    if (row_sum_out)
        memcpy(row_sum_out, S, sizeof(double) * (size_t)R);
    free(S);
    return 0;
}

/* ---- reconstruct: W_eff = W_base + alpha * sign(Delta) ([MF], [SA]) ----- */

static uint16_t weff_at(const uint16_t *w_base, const uint8_t *signs, const float *alpha,
                        int per_matrix, int64_t C, int64_t r, int64_t j)
{
    float a = per_matrix ? alpha[0] : alpha[r];
    float w = oracle_f32_from_bf16(w_base[r * C + j]);
    float e = w + signed_alpha(signs + r * (C / 8), j, a);
    return oracle_bf16_from_f32(e);
}

int oracle_reconstruct(const uint16_t *w_base, const uint8_t *signs, const float *alpha,
                       int per_matrix, int64_t R, int64_t C, uint16_t *w_eff)
{
    if (R < 0 || C <= 0 || C % 8 != 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r)
        for (int64_t j = 0; j < C; ++j)
            w_eff[r * C + j] = weff_at(w_base, signs, alpha, per_matrix, C, r, j);
    return 0;
}

/* ---- linear: y = x W_eff^T in fp64 ([SA] sketch, last line) ------------- */

/* x: bf16 [M, C].  rows: the output rows (W rows) to compute, n_rows of them
 * (NULL means all R rows in order).  y64 out [M, n_rows]; scale out
 * [M, n_rows] = sum_j |x_mj| * |W_eff_rj| (the normaliser of the tolerance).
 * W_eff rows are rebuilt one at a time with the reconstruct formula. */
int oracle_linear_rows(const uint16_t *x, int64_t M, const uint16_t *w_base,
                       const uint8_t *signs, const float *alpha, int per_matrix,
                       int64_t R, int64_t C, const int64_t *rows, int64_t n_rows,
                       double *y64, double *scale)
{
    if (M < 0 || R < 0 || C <= 0 || C % 8 != 0)
        return -1;
    if (!rows)
        n_rows = R;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < n_rows; ++t) {
        int64_t r = rows ? rows[t] : t;
        double *we = (double *)malloc(sizeof(double) * (size_t)C);
        for (int64_t j = 0; j < C; ++j)
            we[j] = (double)oracle_f32_from_bf16(weff_at(w_base, signs, alpha, per_matrix, C, r, j));
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, sc = 0.0;
            for (int64_t j = 0; j < C; ++j) {
                double xv = (double)oracle_f32_from_bf16(x[m * C + j]);
                acc += xv * we[j];
                sc += fabs(xv) * fabs(we[j]);
            }
            y64[m * n_rows + t] = acc;
            if (scale)
                scale[m * n_rows + t] = sc;
        }
        free(we);
    }
    return 0;
}

/* ---- grouped: each token uses its own variant's signs and alpha ---------
 * ([SA] diagram: one HBM-resident W_base read by every variant in the delta
 * cache).  signs [V, R, C/8]; alpha [V, R] (per-row) or [V] (per-matrix).
 * A token whose id is outside [0, V) gets y = 0 and scale = 0.  Columns of
 * the outputs are the W rows listed in `rows` (NULL = all R). */
int oracle_linear_grouped_rows(const uint16_t *x, int64_t M, const int32_t *ids, int32_t V,
                               const uint16_t *w_base, const uint8_t *signs,
                               const float *alpha, int per_matrix, int64_t R, int64_t C,
                               const int64_t *rows, int64_t n_rows,
                               double *y64, double *scale)
{
    if (M < 0 || R < 0 || C <= 0 || C % 8 != 0 || V <= 0)
        return -1;
    if (!rows)
        n_rows = R;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        int32_t v = ids[m];
        for (int64_t t = 0; t < n_rows; ++t) {
            double acc = 0.0, sc = 0.0;
            if (v >= 0 && v < V) {
                int64_t r = rows ? rows[t] : t;
                const uint8_t *sv = signs + (int64_t)v * R * (C / 8);
                const float *av = per_matrix ? alpha + v : alpha + (int64_t)v * R;
                for (int64_t j = 0; j < C; ++j) {
                    double xv = (double)oracle_f32_from_bf16(x[m * C + j]);
                    double w = (double)oracle_f32_from_bf16(weff_at(w_base, sv, av, per_matrix, C, r, j));
                    acc += xv * w;
                    sc += fabs(xv) * fabs(w);
                }
            }
            y64[m * n_rows + t] = acc;
            if (scale)
                scale[m * n_rows + t] = sc;
        }
    }
    return 0;
}

/* ---- similarity of task vectors ([KM] step 1, R7) ----------------------- */

/* signs: [V, R, C/8]; alpha: [V, R] (per_matrix = 0) or [V] (per_matrix = 1).
 * gram, cosv: [V, V] fp64, row-major (both triangles written).
 * Returns 0, or -1 when C is not a positive multiple of 8 or V < 1. */
int oracle_similarity(const uint8_t *signs, const float *alpha, int per_matrix, int32_t V,
                      int64_t R, int64_t C, double *gram, double *cosv)
{
    if (R < 0 || C <= 0 || C % 8 != 0 || V < 1)
        return -1;
    const int64_t G = C / 8;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ab = 0; ab < (int64_t)V * V; ++ab) {
        int32_t a = (int32_t)(ab / V), b = (int32_t)(ab % V);
        if (b < a)
            continue;
        double p[256];
        for (int k = 0; k < 256; ++k)
            p[k] = 0.0;
        for (int64_t r = 0; r < R; ++r) {
            const uint8_t *ra = signs + ((int64_t)a * R + r) * G;
            const uint8_t *rb = signs + ((int64_t)b * R + r) * G;
            int64_t c = 0;
            for (int64_t j = 0; j < C; ++j) {
                int sa = ((ra[j >> 3] >> (j & 7)) & 1) ? 1 : -1;
                int sb = ((rb[j >> 3] >> (j & 7)) & 1) ? 1 : -1;
                c += sa * sb;
            }
            float fa = per_matrix ? alpha[a] : alpha[(int64_t)a * R + r];
            float fb = per_matrix ? alpha[b] : alpha[(int64_t)b * R + r];
            double term = ((double)fa * (double)fb) * (double)c;
            p[r % 256] = p[r % 256] + term;
        }
        double g = halving_tree_256(p);
        gram[(int64_t)a * V + b] = g;
        gram[(int64_t)b * V + a] = g;
    }
    for (int32_t a = 0; a < V; ++a)
        for (int32_t b = 0; b < V; ++b) {
            double na = gram[(int64_t)a * V + a], nb = gram[(int64_t)b * V + b];
            double d = sqrt(na * nb);
            cosv[(int64_t)a * V + b] = d > 0.0 ? gram[(int64_t)a * V + b] / d : 0.0;
        }
    return 0;
}

/* ---- similarity of the full task vectors ([KM] step 1, R9) ------------- */

/* The halving tree over 64 fp64 partial sums (s = 32, 16, ..., 1). */
static double halving_tree_64(double *p)
{
    for (int s = 32; s >= 1; s >>= 1)
        for (int k = 0; k < s; ++k)
            p[k] = p[k] + p[k + s];
    return p[0];
}

/* w_base: bf16 bits [R, C]; w_ft: [V, R, C] fp32 (ft_is_f32 = 1) or bf16
 * bits (0), variant v at offset v*R*C.  gram, cosv: [V, V] fp64 (both
 * triangles).  Returns 0, or -1 when C is not a positive multiple of 8, R is
 * negative or V < 1. */
int oracle_similarity_delta(const uint16_t *w_base, const void *w_ft, int ft_is_f32, int32_t V, int64_t R,
                            int64_t C, double *gram, double *cosv)
{
    if (R < 0 || C <= 0 || C % 8 != 0 || V < 1)
        return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ab = 0; ab < (int64_t)V * V; ++ab) {
        int32_t a = (int32_t)(ab / V), b = (int32_t)(ab % V);
        if (b < a)
            continue;
        double q[256];
        for (int k = 0; k < 256; ++k)
            q[k] = 0.0;
        for (int64_t r = 0; r < R; ++r) {
            double p[64];
            for (int k = 0; k < 64; ++k)
                p[k] = 0.0;
            for (int64_t j = 0; j < C; ++j) {
                float base = oracle_f32_from_bf16(w_base[r * C + j]);
                float da = w_ft_at(w_ft, ft_is_f32, ((int64_t)a * R + r) * C + j) - base;  /* fl32, R3 */
                float db = w_ft_at(w_ft, ft_is_f32, ((int64_t)b * R + r) * C + j) - base;
                double prod = (double)da * (double)db;  /* exact: 24 x 24 significand bits */
                int k = (int)((j / 8) % 64);
                p[k] = p[k] + prod;
            }
            double term = halving_tree_64(p);
            q[r % 256] = q[r % 256] + term;
        }
        double total = halving_tree_256(q);
        gram[(int64_t)a * V + b] = total;
        gram[(int64_t)b * V + a] = total;
    }
    for (int32_t a = 0; a < V; ++a)
        for (int32_t b = 0; b < V; ++b) {
            double norm2 = gram[(int64_t)a * V + a] * gram[(int64_t)b * V + b];
            double den = sqrt(norm2);
            cosv[(int64_t)a * V + b] = den > 0.0 ? gram[(int64_t)a * V + b] / den : 0.0;
        }
    return 0;
}

/* ---- MonoSoup merge ([MS], R8) ------------------------------------------ */

/* One-sided Jacobi (Hestenes) on a matrix M [m, n], m >= n, held by columns
 * (entry (i, j) at A[j*m + i], overwritten): rotate column pairs until every
 * pair is orthogonal to 1e-15 relative; V [n, n], also held by columns (entry
 * (i, j) at V[j*n + i]), accumulates the rotations.  Afterwards column j of
 * A is sigma_j u_j and M = sum_j A[:, j] V[:, j]^T.  Columns whose squared
 * norm is below 1e-30 of the whole matrix's (singular values under 1e-15 of
 * its norm) are left alone. */
static void jacobi_columns(double *A, int64_t m, int64_t n, double *V)
{
    double frob2 = 0.0;
    for (int64_t i = 0; i < m * n; ++i)
        frob2 += A[i] * A[i];
    const double tiny = 1e-30 * frob2;
    for (int64_t i = 0; i < n * n; ++i)
        V[i] = 0.0;
    for (int64_t i = 0; i < n; ++i)
        V[i * n + i] = 1.0;
    for (int sweep = 0; sweep < 80; ++sweep) {
        int rotated = 0;
        for (int64_t p = 0; p < n - 1; ++p)
            for (int64_t q = p + 1; q < n; ++q) {
                double *cp = A + p * m, *cq = A + q * m;
                double alpha = 0.0, beta = 0.0, gamma = 0.0;
                for (int64_t i = 0; i < m; ++i) {
                    double ap = cp[i], aq = cq[i];
                    alpha += ap * ap;
                    beta += aq * aq;
                    gamma += ap * aq;
                }
                if (gamma == 0.0 || alpha <= tiny || beta <= tiny || fabs(gamma) <= 1e-15 * sqrt(alpha * beta))
                    continue;
                rotated = 1;
                double zeta = (beta - alpha) / (2.0 * gamma);
                double tt = (zeta >= 0.0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
                double c = 1.0 / sqrt(1.0 + tt * tt), s = c * tt;
                for (int64_t i = 0; i < m; ++i) {
                    double ap = cp[i], aq = cq[i];
                    cp[i] = c * ap - s * aq;
                    cq[i] = s * ap + c * aq;
                }
                double *vp = V + p * n, *vq = V + q * n;
                for (int64_t i = 0; i < n; ++i) {
                    double xp = vp[i], xq = vq[i];
                    vp[i] = c * xp - s * xq;
                    vq[i] = s * xp + c * xq;
                }
            }
        if (!rotated)
            break;
    }
}

/* w_base: bf16 [R, C]; w_ft: fp32 [k, R, C] (the k checkpoints); rank r in
 * [0, min(R, C)]; out: fp64 [R, C] = W_base + (1/k) sum_i tau_i.
 * sigma (may be NULL): fp64 [k, min(R, C)], each checkpoint's singular
 * values in decreasing order.  A wide task vector (C > R) is decomposed as
 * its transpose (the same singular values, the vectors swapped), so the
 * Jacobi always works on min(R, C) columns.  Returns 0, or -1 on a bad size
 * or no memory. */
int oracle_monosoup(const uint16_t *w_base, const float *w_ft, int32_t k, int64_t R, int64_t C, int32_t r,
                    double *out, double *sigma)
{
    const int64_t n = R < C ? R : C, m = R < C ? C : R;
    const int wide = C > R;
    if (k < 1 || R < 1 || C < 1 || r < 0 || r > n)
        return -1;
    /* tau[ck] holds checkpoint ck's truncation; the checkpoints are
     * independent (one thread each), and their sum below runs in checkpoint
     * order */
    double *tau = malloc(sizeof(double) * (size_t)k * R * C);
    if (!tau)
        return -1;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (int32_t ck = 0; ck < k; ++ck) {
        double *A = malloc(sizeof(double) * m * n), *V = malloc(sizeof(double) * n * n);
        double *norm = malloc(sizeof(double) * n);
        int64_t *order = malloc(sizeof(int64_t) * n);
        if (!A || !V || !norm || !order) {
            free(A); free(V); free(norm); free(order);
            failed = 1;
            continue;
        }
        const float *wi = w_ft + (int64_t)ck * R * C;
        double *tk = tau + (int64_t)ck * R * C;
        /* M = Delta_i [R, C], or its transpose [C, R] when wide, held by
         * columns: M(i, j) at A[j*m + i] */
        for (int64_t i = 0; i < R; ++i)
            for (int64_t c = 0; c < C; ++c) {
                double d = (double)(wi[i * C + c] - oracle_f32_from_bf16(w_base[i * C + c]));
                if (wide)
                    A[i * m + c] = d;
                else
                    A[c * m + i] = d;
            }
        jacobi_columns(A, m, n, V);
        for (int64_t j = 0; j < n; ++j) {
            double s = 0.0;
            for (int64_t i = 0; i < m; ++i)
                s += A[j * m + i] * A[j * m + i];
            norm[j] = sqrt(s);
            order[j] = j;
        }
        /* columns by decreasing singular value (insertion sort, ties by index) */
        for (int64_t a = 1; a < n; ++a) {
            int64_t v = order[a], b = a;
            while (b > 0 && norm[order[b - 1]] < norm[v]) {
                order[b] = order[b - 1];
                --b;
            }
            order[b] = v;
        }
        if (sigma)
            for (int64_t j = 0; j < n; ++j)
                sigma[(int64_t)ck * n + j] = norm[order[j]];
        /* truncation of M = sum over the r largest of A[:, j] V[:, j]^T; tau_i
         * is that, or its transpose when wide */
        for (int64_t i = 0; i < m; ++i)
            for (int64_t c = 0; c < n; ++c) {
                double s = 0.0;
                for (int32_t t = 0; t < r; ++t) {
                    int64_t j = order[t];
                    s += A[j * m + i] * V[j * n + c];
                }
                tk[wide ? c * C + i : i * C + c] = s;
            }
        free(A); free(V); free(norm); free(order);
    }
    if (failed) {
        free(tau);
        return -1;
    }
    for (int64_t i = 0; i < R * C; ++i) {
        double acc = 0.0; /* sum of the tau_i, in checkpoint order */
        for (int32_t ck = 0; ck < k; ++ck)
            acc += tau[(int64_t)ck * R * C + i];
        out[i] = (double)oracle_f32_from_bf16(w_base[i]) + acc / (double)k;
    }
    free(tau);
    return 0;
}

/* Threads the OpenMP runtime will use (reported next to oracle timings). */
#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
void oracle_set_num_threads(int n) { omp_set_num_threads(n); }
#else
int oracle_num_threads(void) { return 1; }
void oracle_set_num_threads(int n) { (void)n; }
#endif

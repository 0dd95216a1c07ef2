// C ABI of the BitDelta library (declared in include/bitdelta.h).
//
// Every argument is checked on the host before anything is launched; a bad
// argument returns a status and launches nothing, so the checks are testable
// on a machine without a GPU.  No call allocates device memory.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <limits>

#include "../../include/bitdelta.h"
#include "bd_launch.h"

namespace {

thread_local char g_err[512] = "";

bd_status fail(bd_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
bd_status fail(bd_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

bd_status device(hipError_t e, const char *what)
{
    if (e == hipSuccess)
        return BD_OK;
    return fail(BD_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int64_t kMaxGrid = std::numeric_limits<int32_t>::max();

bd_status check_matrix(int64_t d_out, int64_t d_in)
{
    if (d_out <= 0)
        return fail(BD_ESHAPE, "d_out must be positive (got %lld)", (long long)d_out);
    if (d_in <= 0 || d_in % 8 != 0)
        return fail(BD_ESHAPE, "d_in must be a positive multiple of 8 (got %lld)", (long long)d_in);
    if (d_out > kMaxGrid || d_in > (int64_t)1 << 40 || d_out > std::numeric_limits<int64_t>::max() / d_in)
        return fail(BD_ESHAPE, "matrix [%lld, %lld] too large", (long long)d_out, (long long)d_in);
    return BD_OK;
}

// The prefill kernels address x, W_base, signs and y through 32-bit buffer
// offsets: each operand (per variant for signs) must stay below 2 GiB.
bool operands_fit(int64_t m, int64_t d_out, int64_t d_in)
{
    // a * b * 2 < 2^31 for positive a, b, without forming the product
    const auto fits = [](int64_t a, int64_t b) { return a <= 0 || b <= 0 || a <= ((int64_t(1) << 30) - 1) / b; };
    return fits(m, d_in) && fits(d_out, d_in) && fits(m, d_out);
}

bd_status check_mode(int mode)
{
    if (mode != BD_ALPHA_ROW && mode != BD_ALPHA_MATRIX)
        return fail(BD_EINVAL, "alpha_mode must be BD_ALPHA_ROW (0) or BD_ALPHA_MATRIX (1), got %d", mode);
    return BD_OK;
}

#define BD_TRY(expr)                  \
    do {                              \
        bd_status s__ = (expr);       \
        if (s__ != BD_OK)             \
            return s__;               \
    } while (0)

#define BD_NONNULL(p)                                             \
    do {                                                          \
        if (!(p))                                                 \
            return fail(BD_EINVAL, "%s must not be NULL", #p);    \
    } while (0)

#define BD_ALIGNED(p, a)                                                        \
    do {                                                                        \
        if (!aligned((p), (a)))                                                 \
            return fail(BD_EALIGN, "%s must be %d-byte aligned", #p, (int)(a)); \
    } while (0)

}  // namespace

extern "C" {

int bitdelta_version(void) { return 100; }

const char *bitdelta_status_string(int s)
{
    switch (s) {
    case BD_OK: return "BD_OK";
    case BD_EINVAL: return "BD_EINVAL: invalid argument";
    case BD_ESHAPE: return "BD_ESHAPE: unsupported or invalid shape";
    case BD_EALIGN: return "BD_EALIGN: misaligned pointer";
    case BD_EWORKSPACE: return "BD_EWORKSPACE: workspace too small";
    case BD_EDEVICE: return "BD_EDEVICE: HIP launch failed";
    case BD_EBUSY: return "BD_EBUSY: no delta-cache slot can be freed";
    default: return "unknown bitdelta status";
    }
}

const char *bitdelta_last_error(void) { return g_err; }

size_t bitdelta_compress_workspace(int64_t d_out, int64_t d_in, int alpha_mode)
{
    (void)d_in;
    if (alpha_mode != BD_ALPHA_MATRIX || d_out <= 0)
        return 0;
    return sizeof(double) * (size_t)d_out;
}

bd_status bitdelta_compress(const bd_bf16 *w_base, const void *w_ft, int ft_dtype, int64_t d_out,
                            int64_t d_in, int alpha_mode, uint8_t *signs, float *alpha,
                            void *workspace, size_t workspace_bytes, void *stream)
{
    BD_TRY(check_mode(alpha_mode));
    if (ft_dtype != BD_BF16 && ft_dtype != BD_F32)
        return fail(BD_EINVAL, "ft_dtype must be BD_BF16 (0) or BD_F32 (1), got %d", ft_dtype);
    BD_TRY(check_matrix(d_out, d_in));
    BD_NONNULL(w_base);
    BD_NONNULL(w_ft);
    BD_NONNULL(signs);
    BD_NONNULL(alpha);
    BD_ALIGNED(w_base, 16);
    BD_ALIGNED(w_ft, 16);
    BD_ALIGNED(alpha, 4);
    const bool per_matrix = alpha_mode == BD_ALPHA_MATRIX;
    const size_t need = bitdelta_compress_workspace(d_out, d_in, alpha_mode);
    if (workspace_bytes < need)
        return fail(BD_EWORKSPACE, "compress needs %zu workspace bytes, got %zu", need, workspace_bytes);
    if (need) {
        BD_NONNULL(workspace);
        BD_ALIGNED(workspace, 8);
    }
    return device(bd::launch_compress(w_base, w_ft, ft_dtype == BD_F32, d_out, d_in, per_matrix, signs,
                                      alpha, static_cast<double *>(workspace), (hipStream_t)stream),
                  "bitdelta_compress");
}

bd_status bitdelta_reconstruct(const bd_bf16 *w_base, const uint8_t *signs, const float *alpha,
                               int alpha_mode, int64_t d_out, int64_t d_in, bd_bf16 *w_eff,
                               void *stream)
{
    BD_TRY(check_mode(alpha_mode));
    BD_TRY(check_matrix(d_out, d_in));
    BD_NONNULL(w_base);
    BD_NONNULL(signs);
    BD_NONNULL(alpha);
    BD_NONNULL(w_eff);
    BD_ALIGNED(w_base, 16);
    BD_ALIGNED(w_eff, 16);
    BD_ALIGNED(alpha, 4);
    const int64_t bpr = (d_in / 8 + 255) / 256;
    if (d_out * bpr > kMaxGrid)
        return fail(BD_ESHAPE, "matrix [%lld, %lld] exceeds the reconstruct grid", (long long)d_out, (long long)d_in);
    return device(bd::launch_reconstruct(w_base, signs, alpha, alpha_mode == BD_ALPHA_MATRIX, d_out, d_in, w_eff,
                                         (hipStream_t)stream),
                  "bitdelta_reconstruct");
}

size_t bitdelta_linear_workspace(int64_t m, int64_t d_out, int64_t d_in)
{
    if (d_out <= 0 || d_in <= 0 || d_in % 8 != 0 || m < 1)
        return 0;
    // decode: only few rows of long width need one (split row steps); shapes
    // the decode path rejects need none
    if (m <= bd::kGemvMaxM)
        return (int64_t)bd::kGemvMaxM * d_in * 2 >= ((int64_t)1 << 31) ? 0 : bd::gemv_workspace_bytes((int)m, d_out, d_in);
    // shapes the prefill path rejects need no workspace
    if (!operands_fit(m, d_out, d_in))
        return 0;
    return bd::gemm_workspace_bytes(m, d_out, d_in);
}

bd_status bitdelta_linear(const bd_bf16 *x, int64_t m, const bd_bf16 *w_base, const uint8_t *signs,
                          const float *alpha, int alpha_mode, int64_t d_out, int64_t d_in, bd_bf16 *y,
                          void *workspace, size_t workspace_bytes, void *stream)
{
    BD_TRY(check_mode(alpha_mode));
    BD_TRY(check_matrix(d_out, d_in));
    if (m < 0)
        return fail(BD_ESHAPE, "m must be >= 0 (got %lld)", (long long)m);
    const size_t need = bitdelta_linear_workspace(m, d_out, d_in);
    if (workspace_bytes < need)
        return fail(BD_EWORKSPACE, "linear needs %zu workspace bytes, got %zu", need, workspace_bytes);
    if (m == 0)
        return BD_OK;
    BD_NONNULL(x);
    BD_NONNULL(w_base);
    BD_NONNULL(signs);
    BD_NONNULL(alpha);
    BD_NONNULL(y);
    BD_ALIGNED(x, 16);
    BD_ALIGNED(w_base, 16);
    BD_ALIGNED(y, 16);
    BD_ALIGNED(alpha, 4);
    if (need) {
        BD_NONNULL(workspace);
        BD_ALIGNED(workspace, 16);
    }
    const bool per_matrix = alpha_mode == BD_ALPHA_MATRIX;
    hipStream_t s = (hipStream_t)stream;
    if (m <= bd::kGemvMaxM) {
        // The decode kernels address x and each launched chunk of W_base (at
        // least 16 rows) through 32-bit buffer offsets.
        if ((int64_t)bd::kGemvMaxM * d_in * 2 >= ((int64_t)1 << 31))
            return fail(BD_ESHAPE, "decode linear needs 16 rows of W_base below 2 GiB (d_in=%lld)", (long long)d_in);
        return device(bd::launch_gemv(x, (int)m, w_base, signs, alpha, per_matrix, d_out, d_in, y, workspace, s),
                      "bitdelta_linear (decode)");
    }
    if (!operands_fit(m, d_out, d_in))
        return fail(BD_ESHAPE, "prefill operands must each be below 2 GiB (m=%lld, d_out=%lld, d_in=%lld)",
                    (long long)m, (long long)d_out, (long long)d_in);
    const int64_t tiles = ((m + bd::kGemmBM - 1) / bd::kGemmBM) * ((d_out + bd::kGemmBN - 1) / bd::kGemmBN);
    if (tiles > kMaxGrid)
        return fail(BD_ESHAPE, "linear m=%lld d_out=%lld exceeds the prefill grid", (long long)m, (long long)d_out);
    if (need >= ((size_t)1 << 31))
        return fail(BD_ESHAPE, "linear m=%lld d_out=%lld d_in=%lld needs a split-K workspace above 2 GiB",
                    (long long)m, (long long)d_out, (long long)d_in);
    return device(bd::launch_gemm(x, m, w_base, signs, alpha, per_matrix, d_out, d_in, y, workspace, s),
                  "bitdelta_linear (prefill)");
}

size_t bitdelta_linear_grouped_workspace(int64_t m, int32_t n_variants, int64_t d_out, int64_t d_in)
{
    (void)d_out;
    (void)d_in;
    if (m < 0 || m > std::numeric_limits<int32_t>::max() / 2 || n_variants <= 0 || n_variants > 4096)
        return 0;
    return bd::grouped_workspace_bytes(m, n_variants);
}

}  // extern "C"

namespace {

// Checks shared by the two grouped entry points (everything but the table's
// memory); BD_OK with *empty set for m = 0, a no-op.
bd_status check_grouped(const bd_bf16 *x, int64_t m, const int32_t *variant_ids, int32_t n_variants,
                        const bd_bf16 *w_base, const uint8_t *signs, const float *alpha, int alpha_mode,
                        int64_t d_out, int64_t d_in, bd_bf16 *y)
{
    BD_TRY(check_mode(alpha_mode));
    if (n_variants <= 0 || n_variants > 4096)
        return fail(BD_EINVAL, "n_variants must be in [1, 4096] (got %d)", n_variants);
    BD_TRY(check_matrix(d_out, d_in));
    if (m < 0)
        return fail(BD_ESHAPE, "m must be >= 0 (got %lld)", (long long)m);
    if (m > std::numeric_limits<int32_t>::max() / 2)
        return fail(BD_ESHAPE, "grouped m=%lld too large for int32 token indices", (long long)m);
    if (m == 0)
        return BD_OK;
    BD_NONNULL(x);
    BD_NONNULL(variant_ids);
    BD_NONNULL(w_base);
    BD_NONNULL(signs);
    BD_NONNULL(alpha);
    BD_NONNULL(y);
    BD_ALIGNED(x, 16);
    BD_ALIGNED(w_base, 16);
    BD_ALIGNED(y, 16);
    BD_ALIGNED(alpha, 4);
    BD_ALIGNED(variant_ids, 4);
    if (!operands_fit(m, d_out, d_in))
        return fail(BD_ESHAPE, "grouped operands must each be below 2 GiB (m=%lld, d_out=%lld, d_in=%lld)",
                    (long long)m, (long long)d_out, (long long)d_in);
    const int64_t tiles = bd::grouped_max_tiles(m, n_variants) * ((d_out + bd::kGemmBN - 1) / bd::kGemmBN);
    if (tiles > kMaxGrid)
        return fail(BD_ESHAPE, "grouped m=%lld d_out=%lld exceeds the grid", (long long)m, (long long)d_out);
    return BD_OK;
}

}  // namespace

extern "C" {

bd_status bitdelta_linear_grouped(const bd_bf16 *x, int64_t m, const int32_t *variant_ids, int32_t n_variants,
                                  const bd_bf16 *w_base, const uint8_t *signs, const float *alpha,
                                  int alpha_mode, int64_t d_out, int64_t d_in, bd_bf16 *y,
                                  void *workspace, size_t workspace_bytes, void *stream)
{
    BD_TRY(check_grouped(x, m, variant_ids, n_variants, w_base, signs, alpha, alpha_mode, d_out, d_in, y));
    const size_t need = bitdelta_linear_grouped_workspace(m, n_variants, d_out, d_in);
    if (workspace_bytes < need)
        return fail(BD_EWORKSPACE, "linear_grouped needs %zu workspace bytes, got %zu", need, workspace_bytes);
    if (m == 0)
        return BD_OK;
    BD_NONNULL(workspace);
    BD_ALIGNED(workspace, 16);
    return device(bd::launch_grouped(x, m, variant_ids, n_variants, w_base, signs, alpha,
                                     alpha_mode == BD_ALPHA_MATRIX, d_out, d_in, y,
                                     static_cast<int32_t *>(workspace), (hipStream_t)stream),
                  "bitdelta_linear_grouped");
}

bd_status bitdelta_linear_grouped_noalloc(const bd_bf16 *x, int64_t m, const int32_t *variant_ids,
                                          int32_t n_variants, const bd_bf16 *w_base, const uint8_t *signs,
                                          const float *alpha, int alpha_mode, int64_t d_out, int64_t d_in,
                                          bd_bf16 *y, void *stream)
{
    static_assert(BD_GROUPED_NOALLOC_MAX_TOKENS == bd::kGroupedNoallocMaxTokens, "token limit");
    BD_TRY(check_grouped(x, m, variant_ids, n_variants, w_base, signs, alpha, alpha_mode, d_out, d_in, y));
    if (m > BD_GROUPED_NOALLOC_MAX_TOKENS)
        return fail(BD_ESHAPE, "linear_grouped_noalloc takes at most %d tokens (got %lld)",
                    BD_GROUPED_NOALLOC_MAX_TOKENS, (long long)m);
    const size_t need = bitdelta_linear_grouped_workspace(m, n_variants, d_out, d_in);
    if (need > bd::grouped_scratch_bytes())
        return fail(BD_ESHAPE, "linear_grouped_noalloc needs %zu table bytes, the library holds %zu", need,
                    bd::grouped_scratch_bytes());
    if (m == 0)
        return BD_OK;
    int32_t *table = nullptr;
    BD_TRY(device(bd::grouped_scratch(&table), "bitdelta_linear_grouped_noalloc (table address)"));
    return device(bd::launch_grouped(x, m, variant_ids, n_variants, w_base, signs, alpha,
                                     alpha_mode == BD_ALPHA_MATRIX, d_out, d_in, y, table, (hipStream_t)stream),
                  "bitdelta_linear_grouped_noalloc");
}

size_t bitdelta_similarity_workspace(int32_t n_variants, int64_t d_out, int64_t d_in)
{
    (void)d_in;
    if (n_variants < 1 || n_variants > bd::kSimilarityMaxVariants)
        return 0;
    return bd::similarity_workspace_bytes(n_variants, d_out);
}

bd_status bitdelta_similarity(const uint8_t *signs, const float *alpha, int alpha_mode, int32_t n_variants,
                              int64_t d_out, int64_t d_in, double *gram, double *cosine, void *workspace,
                              size_t workspace_bytes, void *stream)
{
    BD_TRY(check_mode(alpha_mode));
    if (n_variants < 1 || n_variants > bd::kSimilarityMaxVariants)
        return fail(BD_EINVAL, "n_variants must be in [1, %d] (got %d)", bd::kSimilarityMaxVariants, n_variants);
    BD_TRY(check_matrix(d_out, d_in));
    if (d_in % 32 != 0)
        return fail(BD_ESHAPE, "similarity needs d_in a multiple of 32 (got %lld)", (long long)d_in);
    if ((int64_t)n_variants * d_out * (d_in / 8) >= ((int64_t)1 << 31))
        return fail(BD_ESHAPE, "similarity sign tensor [%d, %lld, %lld] must be below 2 GiB", n_variants,
                    (long long)d_out, (long long)(d_in / 8));
    if ((int64_t)n_variants * (n_variants - 1) / 2 * d_out * 4 >= ((int64_t)1 << 31))
        return fail(BD_ESHAPE, "similarity of %d variants over %lld rows needs pair counts of 2 GiB or more",
                    n_variants, (long long)d_out);
    const size_t need = bitdelta_similarity_workspace(n_variants, d_out, d_in);
    if (workspace_bytes < need)
        return fail(BD_EWORKSPACE, "similarity needs %zu workspace bytes, got %zu", need, workspace_bytes);
    BD_NONNULL(signs);
    BD_NONNULL(alpha);
    BD_NONNULL(gram);
    BD_NONNULL(cosine);
    BD_ALIGNED(signs, 4);
    BD_ALIGNED(alpha, 4);
    BD_ALIGNED(gram, 8);
    BD_ALIGNED(cosine, 8);
    if (need) {
        BD_NONNULL(workspace);
        BD_ALIGNED(workspace, 4);
    }
    return device(bd::launch_similarity(signs, alpha, alpha_mode == BD_ALPHA_MATRIX, n_variants, d_out, d_in, gram,
                                        cosine, static_cast<int32_t *>(workspace), (hipStream_t)stream),
                  "bitdelta_similarity");
}

size_t bitdelta_similarity_delta_workspace(int32_t n_variants, int64_t d_out, int64_t d_in)
{
    (void)d_in;
    if (n_variants < 1 || n_variants > bd::kSimilarityMaxVariants)
        return 0;
    return bd::similarity_delta_workspace_bytes(n_variants, d_out);
}

bd_status bitdelta_similarity_delta(const bd_bf16 *w_base, const void *w_ft, int ft_dtype, int32_t n_variants,
                                    int64_t d_out, int64_t d_in, double *gram, double *cosine, void *workspace,
                                    size_t workspace_bytes, void *stream)
{
    if (ft_dtype != BD_BF16 && ft_dtype != BD_F32)
        return fail(BD_EINVAL, "ft_dtype must be BD_BF16 (0) or BD_F32 (1), got %d", ft_dtype);
    if (n_variants < 1 || n_variants > bd::kSimilarityMaxVariants)
        return fail(BD_EINVAL, "n_variants must be in [1, %d] (got %d)", bd::kSimilarityMaxVariants, n_variants);
    BD_TRY(check_matrix(d_out, d_in));
    const size_t need = bitdelta_similarity_delta_workspace(n_variants, d_out, d_in);
    if (workspace_bytes < need)
        return fail(BD_EWORKSPACE, "similarity_delta needs %zu workspace bytes, got %zu", need, workspace_bytes);
    BD_NONNULL(w_base);
    BD_NONNULL(w_ft);
    BD_NONNULL(gram);
    BD_NONNULL(cosine);
    BD_NONNULL(workspace);
    BD_ALIGNED(w_base, 16);
    BD_ALIGNED(w_ft, 16);
    BD_ALIGNED(gram, 8);
    BD_ALIGNED(cosine, 8);
    BD_ALIGNED(workspace, 8);
    return device(bd::launch_similarity_delta(w_base, w_ft, ft_dtype == BD_F32, n_variants, d_out, d_in, gram, cosine,
                                              static_cast<double *>(workspace), (hipStream_t)stream),
                  "bitdelta_similarity_delta");
}

size_t bitdelta_monosoup_workspace(int64_t rows, int64_t cols, int32_t k, int32_t rank)
{
    const int64_t lim = (int64_t)1 << 21;
    if (rows < 1 || cols < 4 || rows > lim || cols > lim || k < 1 || k > 64 || rank < 0 || rank > bd::kMsL)
        return 0;
    return bd::monosoup_workspace_bytes(rows, cols, k, rank);
}

bd_status bitdelta_monosoup(const bd_bf16 *w_base, const float *w_ft, const float *omega, int32_t k, int64_t rows,
                            int64_t cols, int32_t rank, int32_t power_iters, float *w_merged, double *sigma,
                            void *workspace, size_t workspace_bytes, void *stream)
{
    const int64_t lim = (int64_t)1 << 21;
    if (rows < 1 || cols < 4 || cols % 4 != 0 || rows > lim || cols > lim)
        return fail(BD_ESHAPE, "monosoup needs rows in [1, 2^21] and cols a multiple of 4 in [4, 2^21] (got %lld, %lld)",
                    (long long)rows, (long long)cols);
    if (k < 1 || k > 64)
        return fail(BD_EINVAL, "monosoup needs k in [1, 64] (got %d)", k);
    const int64_t max_rank = rows < cols ? (rows < bd::kMsL ? rows : bd::kMsL) : (cols < bd::kMsL ? cols : bd::kMsL);
    if (rank < 0 || rank > max_rank)
        return fail(BD_EINVAL, "monosoup rank must be in [0, %lld] (got %d)", (long long)max_rank, rank);
    if (power_iters < 0 || power_iters > 256)
        return fail(BD_EINVAL, "monosoup power_iters must be in [0, 256] (got %d)", power_iters);
    const size_t need = bitdelta_monosoup_workspace(rows, cols, k, rank);
    if (workspace_bytes < need)
        return fail(BD_EWORKSPACE, "monosoup needs %zu workspace bytes, got %zu", need, workspace_bytes);
    BD_NONNULL(w_base);
    BD_NONNULL(w_ft);
    BD_NONNULL(w_merged);
    BD_ALIGNED(w_base, 8);
    BD_ALIGNED(w_ft, 16);
    BD_ALIGNED(w_merged, 16);
    if (rank > 0) {
        BD_NONNULL(omega);
        BD_ALIGNED(omega, 16);
    }
    if (sigma)
        BD_ALIGNED(sigma, 8);
    if (need) {
        BD_NONNULL(workspace);
        BD_ALIGNED(workspace, 256);
    }
    return device(bd::launch_monosoup(reinterpret_cast<const uint16_t *>(w_base), w_ft, omega, k, rows, cols, rank,
                                      power_iters, w_merged, sigma, workspace, (hipStream_t)stream),
                  "bitdelta_monosoup");
}

int64_t bitdelta_probe_read_sink_words(int64_t bytes)
{
    if (bytes < 16 || bytes % 16 != 0 || bytes >= ((int64_t)1 << 31))
        return 0;
    return bd::probe_read_sink_words(bytes);
}

bd_status bitdelta_probe_read(const void *src, int64_t bytes, uint32_t *sink, void *stream)
{
    if (bytes < 16 || bytes % 16 != 0 || bytes >= ((int64_t)1 << 31))
        return fail(BD_ESHAPE, "probe_read needs bytes a multiple of 16 in [16, 2^31 - 1] (got %lld)",
                    (long long)bytes);
    BD_NONNULL(src);
    BD_NONNULL(sink);
    BD_ALIGNED(src, 16);
    BD_ALIGNED(sink, 4);
    return device(bd::launch_probe_read(src, bytes, sink, (hipStream_t)stream), "bitdelta_probe_read");
}

bd_status bitdelta_probe_mfma(int32_t blocks, int32_t iters, float a, float b, uint32_t *sink, void *stream)
{
    if (blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 20))
        return fail(BD_ESHAPE, "probe_mfma needs blocks and iters in [1, 2^20] (got %d, %d)", blocks, iters);
    BD_NONNULL(sink);
    BD_ALIGNED(sink, 4);
    return device(bd::launch_probe_mfma(blocks, iters, a, b, sink, (hipStream_t)stream), "bitdelta_probe_mfma");
}

bd_status bitdelta_probe_lds(int32_t blocks, int32_t iters, int32_t mode, int32_t stride, const void *src,
                             int64_t src_bytes, uint32_t *sink, uint64_t *cycles, void *stream)
{
    if (mode < 0 || mode > 3)
        return fail(BD_EINVAL, "probe_lds mode must be 0..3 (got %d)", mode);
    if (blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 16) || stride < 1 || stride > (1 << 20))
        return fail(BD_ESHAPE, "probe_lds needs blocks in [1, 2^20], iters in [1, 2^16], stride in [1, 2^20] "
                               "(got %d, %d, %d)", blocks, iters, stride);
    if (mode == 3) {
        if (src_bytes < 1024 || src_bytes > ((int64_t)1 << 30) || (src_bytes & (src_bytes - 1)) != 0)
            return fail(BD_ESHAPE, "probe_lds mode 3 needs src_bytes a power of two in [1 KB, 1 GiB] (got %lld)",
                        (long long)src_bytes);
        BD_NONNULL(src);
        BD_ALIGNED(src, 16);
    }
    BD_NONNULL(sink);
    BD_NONNULL(cycles);
    BD_ALIGNED(sink, 4);
    BD_ALIGNED(cycles, 8);
    return device(bd::launch_probe_lds(blocks, iters, mode, stride, src, src_bytes, sink, cycles, (hipStream_t)stream),
                  "bitdelta_probe_lds");
}

}  // extern "C"

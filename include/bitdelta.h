/*
 * bitdelta.h -- C ABI of the BitDelta hot path on AMD Instinct MI355X (gfx950).
 *
 * The method: "BitDelta: Serving 14 Zen Models from One GPU Cluster"
 * (hanzo.blog, 2026-02-28), sections "Mathematical Foundation" (task delta
 * Delta = W_ft - W_base, the 1-bit code W_ft ~ W_base + alpha * sign(Delta),
 * alpha = mean |Delta_ij|), "Serving Architecture" (step 3 rebuilds
 * W_eff = W_base + alpha * sign(Delta) inside a fused kernel that never
 * writes W_eff to HBM; the conceptual fused_bitdelta_linear(x, w_base,
 * delta_sign, alpha) sketch; one HBM-resident base read by every variant in
 * the delta cache) and "Infrastructure Details" (signs packed 8 per byte,
 * [4096,4096] -> [4096,512]; alpha stored as fp32, one per output row).
 *
 * Conventions shared by every call:
 *  - Pointers are DEVICE pointers on the current HIP device unless stated.
 *    The caller owns every buffer; the library allocates nothing inside these
 *    calls and keeps no pointer after a call returns.
 *  - bf16 tensors travel as raw 16-bit patterns (bd_bf16).
 *  - Layouts are row-major and dense: W [d_out, d_in], signs [d_out, d_in/8],
 *    x [m, d_in] (a [batch, seq, d_in] activation flattened), y [m, d_out].
 *  - Sign packing: column j of a row is bit (j & 7) of byte (j >> 3) of that
 *    row (least significant bit first); bit 1 means +1, bit 0 means -1; a
 *    delta >= 0 (including -0) is stored as +1.
 *  - alpha: BD_ALPHA_ROW = fp32 [d_out], one per output row;
 *    BD_ALPHA_MATRIX = fp32 [1], one per matrix.
 *  - W_eff[r,j] = bf16_rne(fp32(W_base[r,j]) + (bit ? alpha_r : -alpha_r)),
 *    the sum formed in fp32 and rounded once to bf16 (nearest, ties to even).
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream) and never synchronise the host.  Outputs are fully overwritten
 *    and must not alias inputs.
 *  - Errors are detected on the host before any launch and return a status;
 *    nothing is launched then.  BD_EDEVICE reports a launch failure;
 *    bitdelta_last_error() gives the detail (thread-local).
 *  - Alignment: bf16 and fp32 matrices (x, y, W_base, W_ft, W_eff) must be
 *    16-byte aligned, alpha and variant ids 4-byte aligned, workspaces as
 *    stated per call; signs need no alignment (bitdelta_similarity: 4).
 *  - d_in must be a positive multiple of 8 (whole sign bytes); d_out > 0;
 *    m >= 0 (m = 0 is a no-op returning BD_OK).
 *  - Calls are thread-safe; concurrent calls on different streams may share
 *    read-only inputs.
 */
#ifndef BITDELTA_H
#define BITDELTA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Symbols of the library's C ABI; everything else in it is hidden. */
#ifndef BD_API
#define BD_API __attribute__((visibility("default")))
#endif

typedef uint16_t bd_bf16;

typedef enum {
    BD_OK = 0,
    BD_EINVAL = 1,     /* null pointer with a non-zero extent, bad enum, n_variants <= 0 */
    BD_ESHAPE = 2,     /* d_in % 8 != 0, d_in <= 0, d_out <= 0, m < 0, or a size the grid cannot cover */
    BD_EALIGN = 3,     /* a pointer misses the alignment stated above */
    BD_EWORKSPACE = 4, /* workspace smaller than the matching *_workspace() query */
    BD_EDEVICE = 5,    /* the HIP runtime rejected a launch (delta cache: the loader failed) */
    BD_EBUSY = 6       /* delta cache: no slot can be freed (bitdelta_cache.h) */
} bd_status;

typedef enum { BD_BF16 = 0, BD_F32 = 1 } bd_dtype;

typedef enum { BD_ALPHA_ROW = 0, BD_ALPHA_MATRIX = 1 } bd_alpha_mode;

/* Library version: major * 10000 + minor * 100 + patch. */
BD_API int bitdelta_version(void);

/* Human-readable name of a status code (static string). */
BD_API const char *bitdelta_status_string(int status);

/* Detail of the last non-OK status on this thread (static per thread). */
BD_API const char *bitdelta_last_error(void);

/* ---------------------------------------------------------------- compress
 * "Mathematical Foundation" (Delta, sign, alpha = mean |Delta|) and
 * "Infrastructure Details" (packed sign storage, fp32 alpha per row).
 *
 * Delta[r,j] = fl32(W_ft[r,j] - W_base[r,j]); signs[r, j>>3] bit (j&7) =
 * (Delta >= 0).  alpha: the |Delta| values of a row are summed in fp64 in a
 * fixed order -- 8-column groups g = 0,1,... feed 256 partial sums
 * (group g into partial g mod 256, columns in increasing order), which are
 * then combined by a halving tree (p[k] += p[k+s], s = 128 ... 1).
 *   BD_ALPHA_ROW:    alpha[r] = fp32(S_r / d_in).
 *   BD_ALPHA_MATRIX: the row sums S_r are combined the same way (row r into
 *                    partial r mod 256, then the halving tree) into T, and
 *                    alpha[0] = fp32(T / (d_out * d_in)).
 * w_base: bf16 [d_out, d_in]; w_ft: [d_out, d_in] of type ft_dtype (BD_BF16
 * or BD_F32); signs out: uint8 [d_out, d_in/8]; alpha out: fp32 [d_out] or [1].
 * workspace: device scratch of at least bitdelta_compress_workspace() bytes
 * (0 for BD_ALPHA_ROW; 8 * d_out for BD_ALPHA_MATRIX), 8-byte aligned;
 * may be NULL when the query returns 0. */
BD_API size_t bitdelta_compress_workspace(int64_t d_out, int64_t d_in, int alpha_mode);
BD_API bd_status bitdelta_compress(const bd_bf16 *w_base, const void *w_ft, int ft_dtype,
                            int64_t d_out, int64_t d_in, int alpha_mode,
                            uint8_t *signs, float *alpha,
                            void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------- reconstruct
 * "Serving Architecture", step 3 of the request flow: materialise
 * W_eff = W_base + alpha * sign(Delta) as bf16 [d_out, d_in].  (The fused
 * linear below never does this; this call exists for callers that want the
 * dense weight and as the exact reference of the fused path.) */
BD_API bd_status bitdelta_reconstruct(const bd_bf16 *w_base, const uint8_t *signs, const float *alpha,
                               int alpha_mode, int64_t d_out, int64_t d_in,
                               bd_bf16 *w_eff, void *stream);

/* ------------------------------------------------------------------ linear
 * "Serving Architecture", the fused reconstruct + matmul (the conceptual
 * fused_bitdelta_linear sketch): y = x W_eff^T with W_eff formed in registers
 * and LDS only.  fp32 accumulation, bf16 output (nearest-even).
 * x: bf16 [m, d_in]; y: bf16 [m, d_out].  m <= 16 runs the bandwidth-bound
 * decode kernel; larger m the bf16-MFMA prefill kernel, which needs x, W_base
 * and y each below 2 GiB (BD_ESHAPE otherwise).
 * workspace: at least bitdelta_linear_workspace(m, d_out, d_in) bytes,
 * 16-byte aligned (may be NULL when that is 0).  It is non-zero only for
 * prefill shapes with few 256 x 256 output tiles, whose K loop is split
 * (fp32 partial sums, 256 KB per tile and split), and for decode on 512 to
 * 2048 rows of at least 8192 columns with m >= 5 (or m = 3..4 with x above
 * 64 KB), whose rows are walked in parts (fp32 sums, m * d_out * 4 bytes per
 * part); either way the parts are summed in a fixed order, so the result
 * does not depend on timing.  The caller owns it;
 * its contents are scratch on entry and undefined after the call, and two
 * calls in flight at once must not share one.  Too small: BD_EWORKSPACE; a
 * requirement of 2 GiB or more: BD_ESHAPE. */
BD_API size_t bitdelta_linear_workspace(int64_t m, int64_t d_out, int64_t d_in);
BD_API bd_status bitdelta_linear(const bd_bf16 *x, int64_t m,
                          const bd_bf16 *w_base, const uint8_t *signs, const float *alpha,
                          int alpha_mode, int64_t d_out, int64_t d_in,
                          bd_bf16 *y, void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------- linear_grouped
 * "Serving Architecture", the delta cache: many variants share one
 * HBM-resident W_base; token i uses variant v = variant_ids[i]:
 *   y[i] = x[i] (W_base + alpha_v * sign(Delta_v))^T.
 * variant_ids: int32 [m] on the device; ids outside [0, n_variants) give a
 * zero row.  signs: uint8 [n_variants, d_out, d_in/8]; alpha: fp32
 * [n_variants, d_out] (BD_ALPHA_ROW) or [n_variants] (BD_ALPHA_MATRIX).
 * Tokens are bucketed by variant on the device (no host synchronisation).
 * n_variants must be in [1, 4096]; x, W_base, y and each variant's signs
 * must be below 2 GiB (BD_ESHAPE otherwise).
 * workspace: at least bitdelta_linear_grouped_workspace() bytes, 16-byte
 * aligned. */
BD_API size_t bitdelta_linear_grouped_workspace(int64_t m, int32_t n_variants, int64_t d_out, int64_t d_in);
BD_API bd_status bitdelta_linear_grouped(const bd_bf16 *x, int64_t m, const int32_t *variant_ids,
                                  int32_t n_variants, const bd_bf16 *w_base,
                                  const uint8_t *signs, const float *alpha, int alpha_mode,
                                  int64_t d_out, int64_t d_in, bd_bf16 *y,
                                  void *workspace, size_t workspace_bytes, void *stream);

/* -------------------------------------------------- linear_grouped_noalloc
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * operation, arguments and results as bitdelta_linear_grouped, with the
 * bucketing table kept in an array of the library in device memory instead
 * of a caller workspace.  Each GPU the library runs on holds its own copy
 * (about 307 KiB, until the process ends); its address is looked up once per
 * device, on the first call made with that device current.  The call
 * allocates nothing and needs nothing cleared: every call rewrites the
 * table.  All calls on one GPU share that table, so calls that overlap in
 * time on one GPU (on different streams, or from different threads without
 * ordering) race and give undefined results; calls ordered on one stream are
 * safe.  m at most BD_GROUPED_NOALLOC_MAX_TOKENS (BD_ESHAPE otherwise);
 * every other check and error as in bitdelta_linear_grouped. */
#define BD_GROUPED_NOALLOC_MAX_TOKENS 65536
BD_API bd_status bitdelta_linear_grouped_noalloc(const bd_bf16 *x, int64_t m, const int32_t *variant_ids,
                                          int32_t n_variants, const bd_bf16 *w_base,
                                          const uint8_t *signs, const float *alpha, int alpha_mode,
                                          int64_t d_out, int64_t d_in, bd_bf16 *y, void *stream);

/* -------------------------------------------------------------- similarity
 * "K-Merge: Online LoRA Adapter Management for the Edge", step 1 of the
 * pool policy: the cosine similarity of two variants' task vectors.  The task
 * vector of variant v over one matrix is its BitDelta delta
 * tau_v[r][j] = alpha_v[r] * s_v[r][j] (s = +1 for bit 1, -1 for bit 0).
 * Outputs, host-readable after the stream completes (fp64, [n_variants,
 * n_variants] row-major, both triangles):
 *   gram[a][b]   = <tau_a, tau_b>, summed in a fixed order: per row r the
 *                  integer c = sum_j s_a s_b (exact), the term
 *                  (alpha_a[r] * alpha_b[r]) * c in fp64 (one rounding);
 *                  row r into partial r mod 256 in increasing r, then the
 *                  halving tree p[k] += p[k + s], s = 128 .. 1.  The same
 *                  bits on every call and every GPU.
 *   cosine[a][b] = gram[a][b] / sqrt(gram[a][a] * gram[b][b]) (0 when a
 *                  norm is 0).
 * signs: uint8 [n_variants, d_out, d_in/8], 4-byte aligned, with d_in a
 * multiple of 32 (4-byte aligned sign rows) and n_variants * d_out * d_in/8
 * below 2 GiB (BD_ESHAPE otherwise); alpha: fp32 [n_variants, d_out]
 * (BD_ALPHA_ROW) or [n_variants] (BD_ALPHA_MATRIX); n_variants in [1, 16]
 * (BD_EINVAL otherwise).  gram and cosine: device fp64 [n_variants^2],
 * 8-byte aligned.
 * workspace: at least bitdelta_similarity_workspace() bytes (int32 per row
 * and pair of variants; 0 for one variant), 4-byte aligned; owned by the
 * caller, scratch on entry, undefined after; calls in flight at once must
 * not share one. */
BD_API size_t bitdelta_similarity_workspace(int32_t n_variants, int64_t d_out, int64_t d_in);
BD_API bd_status bitdelta_similarity(const uint8_t *signs, const float *alpha, int alpha_mode,
                              int32_t n_variants, int64_t d_out, int64_t d_in,
                              double *gram, double *cosine,
                              void *workspace, size_t workspace_bytes, void *stream);

/* -------------------------------------------------------- similarity_delta
 * "K-Merge: Online LoRA Adapter Management for the Edge", step 1 of the pool
 * policy (the cosine similarity of two adapters' task vectors), with the task
 * vector of section "MonoSoup": the fine-tuned weights minus the base
 * weights.  For n_variants fine-tuned copies W_ft_v of one matrix,
 * Delta_v[r][j] = fl32(W_ft_v[r][j] - W_base[r][j]) (the same fp32 difference
 * as bitdelta_compress).  Outputs (fp64 [n_variants, n_variants], row-major,
 * both triangles, device, 8-byte aligned):
 *   gram[a][b]   = <Delta_a, Delta_b>, summed in a fixed order: per row r the
 *                  products Delta_a Delta_b (exact in fp64) of 8-column group
 *                  g go into partial g mod 64 (columns and groups in
 *                  increasing order), the 64 partials are combined by the
 *                  halving tree p[k] += p[k + s], s = 32 .. 1; the row terms
 *                  then go into partial r mod 256 in increasing r, combined
 *                  by the halving tree s = 128 .. 1.  The same bits on every
 *                  call and every GPU.
 *   cosine[a][b] = gram[a][b] / sqrt(gram[a][a] * gram[b][b]) (0 when a
 *                  norm is 0).
 * w_base: bf16 [d_out, d_in]; w_ft: [n_variants, d_out, d_in] of type
 * ft_dtype (BD_BF16 or BD_F32), variant v at element offset v*d_out*d_in;
 * both 16-byte aligned.  n_variants in [1, 16] (BD_EINVAL otherwise).
 * Unlike bitdelta_similarity this reads the full-precision weights (HBM-bound
 * on W_ft); it needs no compressed code.
 * workspace: at least bitdelta_similarity_delta_workspace() bytes (fp64 per
 * row and pair of variants, diagonal included), 8-byte aligned; owned by the
 * caller, scratch on entry, undefined after; calls in flight at once must
 * not share one. */
BD_API size_t bitdelta_similarity_delta_workspace(int32_t n_variants, int64_t d_out, int64_t d_in);
BD_API bd_status bitdelta_similarity_delta(const bd_bf16 *w_base, const void *w_ft, int ft_dtype,
                                    int32_t n_variants, int64_t d_out, int64_t d_in,
                                    double *gram, double *cosine,
                                    void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------- MonoSoup
 * "BitDelta: Serving 14 Zen Models from One GPU Cluster", section "MonoSoup":
 * k fine-tuned checkpoints W_1..W_k of one matrix are merged through the
 * rank-r truncated SVD tau_i of each task vector Delta_i = W_i - W_base:
 *   W_merged = W_base + (1/k) sum_i tau_i.
 * Delta_i is the fp32 difference fl32(W_i - f32(W_base)).  The truncation is
 * computed by a randomized range finder with a sketch of
 * BD_MONOSOUP_SKETCH (64) columns: Y = Delta Omega, then power_iters rounds
 * of Y <- Delta (Delta^T Y) with the sketch re-orthonormalised between
 * products, then the exact rank-r truncation of the projection of Delta onto
 * range(Y).  It equals the exact truncated SVD (up to fp32 rounding) when
 * Delta has rank at most 64.  Otherwise its relative distance from it is at
 * most about sqrt(2) t0 (sigma_65 / sigma_r)^(2 power_iters + 1)
 * sigma_1 / sigma_r in exact arithmetic (t0 = ||(V_rest^T Omega)(V_64^T
 * Omega)^-1||_2, V_64 the 64 leading right singular vectors of Delta) plus
 * fp32 rounding, which grows as sigma_r approaches sigma_{r+1}: a spectrum
 * that drops after the r-th value needs one or two rounds, a flat one (a
 * random Laplace delta: sigma_65 / sigma_32 about 0.93) one to two hundred.
 * Each round costs two passes over the k task vectors and two whitenings.
 *   w_base: bf16 [rows, cols], 8-byte aligned.
 *   w_ft:   fp32 [k, rows, cols] (checkpoint i at offset i*rows*cols),
 *           16-byte aligned.
 *   omega:  fp32 [cols, 64], 16-byte aligned: the test matrix, normally
 *           i.i.d. N(0, 1) drawn by the caller (unused, may be NULL, when
 *           rank is 0).
 *   rank:   r in [0, min(64, rows, cols)]; power_iters in [0, 256]
 *           (BD_EINVAL otherwise); k in [1, 64] (BD_EINVAL).
 *   rows >= 1, cols >= 4 a multiple of 4, both at most 2^21 (BD_ESHAPE).
 *   w_merged: fp32 [rows, cols], 16-byte aligned: f32(W_base) + the fp32
 *           contraction of the k rank-r factors.
 *   sigma:  NULL, or fp64 [k, rank], 8-byte aligned: the estimated leading
 *           singular values of each Delta_i, decreasing.
 * workspace: at least bitdelta_monosoup_workspace() bytes (0 for rank 0),
 * 256-byte aligned; owned by the caller, scratch on entry, undefined after;
 * calls in flight at once must not share one.  The result is deterministic
 * (every reduction runs in a fixed order). */
#define BD_MONOSOUP_SKETCH 64
BD_API size_t bitdelta_monosoup_workspace(int64_t rows, int64_t cols, int32_t k, int32_t rank);
BD_API bd_status bitdelta_monosoup(const bd_bf16 *w_base, const float *w_ft, const float *omega,
                            int32_t k, int64_t rows, int64_t cols, int32_t rank, int32_t power_iters,
                            float *w_merged, double *sigma,
                            void *workspace, size_t workspace_bytes, void *stream);

/* -------------------------------------------------------------- probes
 * Measurement utilities with no counterpart in the method: they give the
 * practical streaming-read rate, dense bf16 MFMA rate and LDS rates of the
 * device, so the method's kernels can be read against what the chip sustains
 * as well as against its published peaks.
 *
 * bitdelta_probe_read: reads `bytes` bytes at `src` once (16-byte streaming
 * loads, one 1 KB contiguous run per 64-lane instruction) and writes one
 * 32-bit word per wave to `sink`: the XOR of every 32-bit word the wave
 * read, so the XOR of all sink words is the XOR of the whole buffer.
 *   src:   device, 16-byte aligned; bytes a multiple of 16 in [16, 2^31 - 1]
 *          (BD_ESHAPE otherwise).
 *   sink:  device, 4-byte aligned, bitdelta_probe_read_sink_words(bytes)
 *          words (0 for an invalid size), fully overwritten.
 * bitdelta_probe_mfma: `blocks` workgroups of 4 waves; each wave runs `iters`
 * rounds of 8 independent v_mfma_f32_32x32x16_bf16 (32 x 32 x 16 bf16
 * products, fp32 accumulation) on register operands whose every element is
 * bf16(a) (A) and bf16(b) (B), then writes to sink[wave] the fp32 bits of the
 * sum over its 8 accumulators of lane 0's first element: 8 * 16 * iters *
 * bf16(a) * bf16(b) (exact while that stays below 2^24 ulps).  flop =
 * blocks * 4 * iters * 8 * 32768.
 *   blocks in [1, 2^20], iters in [1, 2^20] (BD_ESHAPE otherwise); sink:
 *   device, 4-byte aligned, blocks * 4 words. */
BD_API int64_t bitdelta_probe_read_sink_words(int64_t bytes);
BD_API bd_status bitdelta_probe_read(const void *src, int64_t bytes, uint32_t *sink, void *stream);
BD_API bd_status bitdelta_probe_mfma(int32_t blocks, int32_t iters, float a, float b, uint32_t *sink,
                                     void *stream);

/* bitdelta_probe_lds: the LDS rates the kernels' on-chip staging is made of.
 * `blocks` workgroups of 16 waves, one per CU (each declares 96 KB of LDS);
 * each fills 64 KB of LDS with word i = i * 0x9E3779B1 (mod 2^32), then every
 * wave w issues 8 * iters operations u = 0, 1, ..., each moving one
 * contiguous block without bank conflicts:
 *   mode 0: ds_read_b128 of the 1 KB block (u * stride + w) mod 64;
 *   mode 1: ds_read_b64 of the 512-byte block (u * stride + w) mod 128;
 *   mode 2: ds_write_b128 of 1 KB into block 4w + (u mod 4), lane l writing
 *           the words u * 0x9E3779B1 + l, (u << 8) ^ l, u + l * 0x01000193,
 *           ~(u ^ (l << 16)) (all mod 2^32);
 *   mode 3: a direct-to-LDS copy (16 bytes per lane) of the 1 KB block
 *           (u * stride + w) mod (src_bytes / 1024) of src into block
 *           4w + (u mod 4).
 * cycles[b] = shader-clock cycles of workgroup b between a barrier before the
 * first operation and one after the last has completed;
 * sink[b * 16 + w] = the XOR of every 32-bit word wave w read (modes 0, 1) or
 * of the final content of its blocks 4w .. 4w + 3 (modes 2, 3).
 *   mode in [0, 3] (BD_EINVAL); blocks in [1, 2^20], iters in [1, 2^16],
 *   stride in [1, 2^20] (BD_ESHAPE); mode 3: src device, 16-byte aligned,
 *   src_bytes a power of two in [1024, 2^30] (BD_ESHAPE), otherwise unused.
 *   sink: device, 4-byte aligned, blocks * 16 words; cycles: device,
 *   8-byte aligned, blocks words. */
BD_API bd_status bitdelta_probe_lds(int32_t blocks, int32_t iters, int32_t mode, int32_t stride, const void *src,
                                    int64_t src_bytes, uint32_t *sink, uint64_t *cycles, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BITDELTA_H */

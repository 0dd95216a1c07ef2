// Host-side launchers of the gfx950 kernels (called by the C ABI in api.cpp
// after all argument checks).  Each returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bd {

// compress.hip
hipError_t launch_compress(const uint16_t *w_base, const void *w_ft, bool ft_f32, int64_t d_out,
                           int64_t d_in, bool per_matrix, uint8_t *signs, float *alpha,
                           double *row_sums, hipStream_t s);

// reconstruct.hip
hipError_t launch_reconstruct(const uint16_t *w_base, const uint8_t *signs, const float *alpha,
                              bool per_matrix, int64_t d_out, int64_t d_in, uint16_t *w_eff,
                              hipStream_t s);

// gemv.hip: m in [1, 16]
constexpr int kGemvMaxM = 16;
// Few rows of long width split the row's steps over more workgroups; their
// fp32 partial sums need gemv_workspace_bytes() of workspace (0 otherwise).
int gemv_splits(int m, int64_t rows, int64_t d_in);
size_t gemv_workspace_bytes(int m, int64_t rows, int64_t d_in);
hipError_t launch_gemv(const uint16_t *x, int m, const uint16_t *w_base, const uint8_t *signs,
                       const float *alpha, bool per_matrix, int64_t d_out, int64_t d_in,
                       uint16_t *y, void *workspace, hipStream_t s);

// gemm.hip: dense prefill GEMM and the grouped variant
constexpr int kGemmBM = 256;
constexpr int kGemmBN = 256;
constexpr int kGemmBNNarrow = 128;
// How a call is cut: tiles kGemmBM x tn, every tile's K loop in `splits`
// ranges, or (tail > 0) the last `tail` tiles in a second launch with K in
// `tail_splits` ranges.
struct GemmPlan {
    int splits;
    int64_t tail;
    int tail_splits;
    int tn;
};
GemmPlan gemm_plan(int64_t m, int64_t d_out, int64_t d_in);
int64_t gemm_k_split(int64_t d_in, int splits);
// `workspace` must hold gemm_workspace_bytes(m, d_out, d_in) bytes (split-K
// partials; 0 when the shape runs unsplit).
size_t gemm_workspace_bytes(int64_t m, int64_t d_out, int64_t d_in);
hipError_t launch_gemm(const uint16_t *x, int64_t m, const uint16_t *w_base, const uint8_t *signs,
                       const float *alpha, bool per_matrix, int64_t d_out, int64_t d_in,
                       uint16_t *y, void *workspace, hipStream_t s);

// Grouped: bucketing writes this table into the workspace, then the grouped
// GEMM walks it.  Layout (int32 words): [0] total tiles, [1..3] pad,
// then perm[m], tile_v[max_tiles], tile_row0[max_tiles], tile_rows[max_tiles].
int64_t grouped_max_tiles(int64_t m, int32_t n_variants);
size_t grouped_workspace_bytes(int64_t m, int32_t n_variants);
hipError_t launch_grouped(const uint16_t *x, int64_t m, const int32_t *ids, int32_t n_variants,
                          const uint16_t *w_base, const uint8_t *signs, const float *alpha,
                          bool per_matrix, int64_t d_out, int64_t d_in, uint16_t *y,
                          int32_t *workspace, hipStream_t s);
// The same table in a device-resident array of the library (one per GPU, no
// allocation), for calls of at most kGroupedNoallocMaxTokens tokens:
// grouped_scratch() gives the current device's copy.
constexpr int64_t kGroupedNoallocMaxTokens = 65536;
size_t grouped_scratch_bytes();
hipError_t grouped_scratch(int32_t **table);

// similarity.hip: Gram matrix and cosines of up to kSimilarityMaxVariants
// variants' task vectors; `counts` holds similarity_workspace_bytes() bytes
// (int32 per row and pair).
constexpr int kSimilarityMaxVariants = 16;
size_t similarity_workspace_bytes(int32_t n_variants, int64_t d_out);
hipError_t launch_similarity(const uint8_t *signs, const float *alpha, bool per_matrix, int32_t n_variants,
                             int64_t d_out, int64_t d_in, double *gram, double *cosine, int32_t *counts,
                             hipStream_t s);

// similarity_delta.hip: Gram matrix and cosines of up to
// kSimilarityMaxVariants variants' full task vectors W_ft - W_base; `terms`
// holds similarity_delta_workspace_bytes() bytes (fp64 per row and pair,
// diagonal included).
size_t similarity_delta_workspace_bytes(int32_t n_variants, int64_t d_out);
hipError_t launch_similarity_delta(const uint16_t *w_base, const void *w_ft, bool ft_f32, int32_t n_variants,
                                   int64_t d_out, int64_t d_in, double *gram, double *cosine, double *terms,
                                   hipStream_t s);

// monosoup.hip: MonoSoup merge through a 64-column randomized range finder.
constexpr int kMsL = 64;
size_t monosoup_workspace_bytes(int64_t rows, int64_t cols, int32_t k, int32_t rank);
hipError_t launch_monosoup(const uint16_t *w_base, const float *w_ft, const float *omega, int32_t k,
                           int64_t rows, int64_t cols, int32_t rank, int32_t power_iters, float *out,
                           double *sigma, void *workspace, hipStream_t s);

// probe.hip: measurement probes (no part of the method).  probe_read reads
// `bytes` (a multiple of 16, below 2 GiB) and writes
// probe_read_sink_words(bytes) words; probe_mfma writes blocks * 4 words.
int64_t probe_read_sink_words(int64_t bytes);
hipError_t launch_probe_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t s);
hipError_t launch_probe_mfma(int32_t blocks, int32_t iters, float a, float b, uint32_t *sink, hipStream_t s);
// probe_lds writes blocks * 16 sink words and blocks cycle counts; mode 3
// reads src (src_bytes a power of two from 1 KB to 1 GiB).
hipError_t launch_probe_lds(int32_t blocks, int32_t iters, int32_t mode, int32_t stride, const void *src,
                            int64_t src_bytes, uint32_t *sink, uint64_t *cycles, hipStream_t s);

}  // namespace bd

// Decode kernels: fused BitDelta linear for m <= 16 tokens.
//
// "BitDelta: Serving 14 Zen Models from One GPU Cluster", section "Serving
// Architecture": the fused kernel reads the base weights and the packed
// delta bits together and builds the effective weight in registers, never
// writing W_eff to HBM (the conceptual fused_bitdelta_linear sketch gives the
// semantics y = x (W_base + alpha * unpack(signs))^T).
//
// At m <= 16 the layer is bound by HBM bandwidth (1 to 15 flop per byte of
// W_base + signs); the kernels exist to keep enough bytes in flight with as
// few memory instructions as possible, and to keep the arithmetic per weight
// small enough to hide under the loads.  Both build W_eff = bf16(W_base +
// s alpha) the same way: the sign nibbles index a 16-entry LDS table of four
// +-1.0f, one fma per weight (s alpha is exact, so the fma rounds once, as
// the add would) and one v_cvt_pk_bf16_f32 per pair.
//
//  gemv_stream (m <= 4, vector ALU; workgroups of 4 waves at m = 1, 8
//    otherwise): a wave owns RW rows and walks them 512
//    columns per step; lane l loads the 16 bytes of columns 8l..8l+7 of each
//    row (every load instruction is 1 KB of one row, streamed past the
//    caches), its sign byte, and the same columns of each token of x (L2
//    hits; at m = 2..4 with x of at most 64 KB, from a copy of x made once
//    per workgroup in LDS; at m = 3..4 with a larger x and d_in a multiple
//    of 4096, gemv_rows instead: read from L2 per wave, x would cost 4 times
//    the weights' bytes).  A ring of D register stages keeps D steps of
//    loads in flight;
//    the loop is a steady part (consume a stage, refill it D steps ahead) and
//    a drain, every address valid or deliberately out of range, so no load
//    sits under a branch, and scheduling barriers keep the loads in issue
//    order so the compiler's waits leave the later stages in flight.  Each
//    packed W_eff pair meets every token in one v_dot2_f32_bf16; the RW * m
//    per-lane sums are reduced across the wave by a reduce-scatter.
//
//  gemv_rows (m in 5..16, and 3..4 with x above 64 KB; d_in a multiple of
//    4096; matrix cores): the memory side of gemv_stream at m = 1 -- each of
//    16 waves streams one or two whole rows, 1 KB per load -- with the token
//    products on MFMA after a transpose of the workgroup's 16 or 32 rows of
//    W_eff through LDS (its own comment below).
//
//  gemv_mfma (m in 5..16, other d_in): one workgroup of 8 waves per block of
//    16 rows; the columns are cut into super-blocks of 128 and wave w takes
//    super-blocks w, w + 8, ...  Lane l (j = l % 16, q = l / 16) loads, for
//    MFMA jj, the 16 bytes of chunk 4jj + q of row n0 + j (so the 4 lanes of a
//    row read 64 contiguous bytes per instruction) and the same columns of
//    token j, and runs v_mfma_f32_16x16x32_bf16 with A = x (tokens x 32
//    columns) and B = W_eff (32 columns x rows).  A and B lanes of one q hold
//    the same columns, whatever order the MFMA takes its k slots in.  Two
//    register stages are in flight; the 8 partial 16 x 16 tiles are summed
//    through LDS in wave order.
//
// All sums are in a fixed order: results do not depend on timing.
#include <algorithm>
#include <type_traits>

#include "bd_device.h"
#include "bd_launch.h"

namespace bd {
namespace {

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

// ------------------------------------------------------------------ m <= 4
// EVEN: d_in / 8 is a multiple of 64 (no ragged last step).  S = the number of
// 512-column steps is a multiple of D (the host picks D).  XL (EVEN only): x
// is copied once into the workgroup's LDS (dynamic, m * d_in * 2 bytes) by
// direct-to-LDS loads issued ahead of the first weight stages, and every wave
// reads its token columns from there instead of from L2 (at m = 4 the L2 reads
// of x are otherwise twice those of W_base).
// Waves per workgroup of gemv_stream: 4 at m = 1 (1024 workgroups on a
// 4096-row layer measured 2.2% faster than 512 of 8 waves), 8 otherwise.
template <int MT>
constexpr int stream_waves() { return MT == 1 ? 4 : 8; }

template <int MT, int RW, int D, bool PER_MATRIX, bool EVEN, bool XL>
__global__ __launch_bounds__(512) void gemv_stream(const uint16_t *__restrict__ x, int m,
                                                   const uint16_t *__restrict__ w_base,
                                                   const uint8_t *__restrict__ signs,
                                                   const float *__restrict__ alpha, int64_t R, int64_t K,
                                                   uint16_t *__restrict__ y, int64_t ldy)
{
    constexpr int kWaves = stream_waves<MT>();
    static_assert(!XL || EVEN, "x in LDS needs whole 512-column steps");
    __shared__ __attribute__((aligned(16))) float sgn[64];
    extern __shared__ __attribute__((aligned(16))) uint8_t xs[];  // XL: x [m, K] bf16
    fill_sign_table(sgn);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row0 = ((int64_t)blockIdx.x * kWaves + wave) * RW;
    const int64_t G = K >> 3;
    const int S = (int)((G + 63) >> 6);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w_base, R * K * 2);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(signs, R * G);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (int64_t)m * K * 2);
    if constexpr (XL) {
        // 1 KB chunk c of x (flat [m, K], a whole number of chunks since K is
        // a multiple of 512) -> LDS bytes [1024 c, +1024): wave w copies
        // chunks w, w + kWaves, ...  The host bounds m * K * 2 by 64 KB, so
        // a wave has at most 64 / kWaves of these in flight.
        const int chunks = (int)(((int64_t)m * K * 2) >> 10);
        for (int c = wave; c < chunks; c += kWaves)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(xs + c * 1024), 16, (uint32_t)(16 * lane),
                                                     (uint32_t)(c * 1024), 0, 0);
        __builtin_amdgcn_sched_barrier(0);  // the copies stay ahead of the weight loads
    }
    // Rows past R use an out-of-range lane offset (zeros, never stored).
    // The scalar offset of a load (the step's column offset) is outside the
    // hardware range check, so it only ever moves within a row whose lane
    // offset is valid: in a ragged last step the lanes past the row use the
    // out-of-range offset for W_base, the sign byte and x alike (zeros).
    uint32_t wrow[RW], srow[RW];
    float a[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const bool ok = row0 + r < R;
        wrow[r] = ok ? (uint32_t)((row0 + r) * K * 2 + 16 * lane) : kInvalidOffset;
        srow[r] = ok ? (uint32_t)((row0 + r) * G + lane) : kInvalidOffset;
        a[r] = PER_MATRIX ? alpha[0] : alpha[ok ? row0 + r : R - 1];
    }
    uint32_t xrow[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
        xrow[t] = t < m ? (uint32_t)(t * K * 2 + 16 * lane) : kInvalidOffset;

    uint4 wq[D][RW], xq[D][MT];
    uint32_t sq[D][RW];
    auto load = [&](int d, int s) {
        bool live = true;
        if constexpr (!EVEN)
            live = (int64_t)s * 64 + lane < G;
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            wq[d][r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     rw, live ? wrow[r] : kInvalidOffset, (uint32_t)s * 1024u, kStream));
            sq[d][r] = __builtin_amdgcn_raw_buffer_load_b8(rs, live ? srow[r] : kInvalidOffset, (uint32_t)s * 64u,
                                                           kStream);
        }
        if constexpr (!XL) {
#pragma unroll
            for (int t = 0; t < MT; ++t)
                xq[d][t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                         rx, live ? xrow[t] : kInvalidOffset, (uint32_t)s * 1024u, 0));
        }
    };
    float acc[RW * MT];
#pragma unroll
    for (int i = 0; i < RW * MT; ++i)
        acc[i] = 0.0f;
    auto compute = [&](int d, int s) {
        if constexpr (XL) {
            // tokens past m read LDS rows that hold nothing useful; their sums
            // are never stored
#pragma unroll
            for (int t = 0; t < MT; ++t)
                xq[d][t] = *reinterpret_cast<const uint4 *>(xs + ((int64_t)(t < m ? t : 0) * K * 2 + s * 1024 + 16 * lane));
        }
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const uint4 e = weff8(sgn, sq[d][r], wq[d][r], a[r]);
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
    for (int d = 0; d < D; ++d) {
        load(d, d);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (XL) {
        // the x copies were issued before the 2 * RW * D loads of the first
        // stages: once at most that many are outstanding, this wave's copies
        // have landed; the barrier makes every wave's visible
        wait_vmcnt<2 * RW * D>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int s0 = 0; s0 < S - D; s0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            compute(d, s0 + d);
            __builtin_amdgcn_sched_barrier(0);
            load(d, s0 + d + D);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
        compute(d, S - D + d);

    constexpr int N = RW * MT;
    constexpr int kbits = log2i<N>();
    const float v = wave_reduce_scatter<N>(acc);
    const int idx = lane >> (6 - kbits);
    if ((lane & ((1 << (6 - kbits)) - 1)) == 0) {
        const int r = idx / MT, t = idx - r * MT;
        if (row0 + r < R && t < m)
            y[(int64_t)t * ldy + row0 + r] = to_bf16(v);
    }
}

// ------------------------------------------------------------- m in 5..16
constexpr int kMfmaWaves = 8;


constexpr int kSuperK = 128;  // columns per super-block (4 MFMA chunks of 32)

// EVEN: d_in is a multiple of 128 (whole super-blocks; sign rows 16-byte
// aligned, so each lane fetches its super-block's 16 sign bytes in one
// 16-byte load).  Otherwise the lane loads its 4 sign bytes one by one and
// x is zero past the row.
template <bool PER_MATRIX, bool EVEN>
__global__ __launch_bounds__(64 * kMfmaWaves) void gemv_mfma(const uint16_t *__restrict__ x, int m,
                                                             const uint16_t *__restrict__ w_base,
                                                             const uint8_t *__restrict__ signs,
                                                             const float *__restrict__ alpha, int64_t R,
                                                             int64_t K, uint16_t *__restrict__ y, int64_t ldy)
{
    constexpr int KW = kMfmaWaves;
    constexpr int JJ = kSuperK / 32;  // MFMAs per super-block
    __shared__ __attribute__((aligned(16))) float sgn[64];
    __shared__ f32x4 red[KW][64];
    fill_sign_table(sgn);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 15, q = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t G = K >> 3;
    const int T = (int)((K + kSuperK - 1) / kSuperK);
    const int nt = T > wave ? (T - 1 - wave) / KW + 1 : 0;  // this wave's super-blocks (uniform)
    const bool row_ok = n0 + j < R;
    const float a = PER_MATRIX ? alpha[0] : alpha[row_ok ? n0 + j : R - 1];
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w_base, R * K * 2);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(signs, R * G);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (int64_t)m * K * 2);
    const uint32_t wrow = row_ok ? (uint32_t)((n0 + j) * K * 2 + 16 * q) : kInvalidOffset;
    const uint32_t srow = row_ok ? (uint32_t)((n0 + j) * G) : kInvalidOffset;
    const uint32_t xrow = j < m ? (uint32_t)(j * K * 2 + 16 * q) : kInvalidOffset;

    struct Stage {
        uint4 w[JJ], x[JJ];
        uint32_t s[JJ];  // EVEN: the 16 sign bytes (dword jj holds chunk 4jj + q in byte q); else byte jj
    };
    Stage st[2];
    // Stages past the wave's last super-block are issued with out-of-range
    // offsets: no traffic, and zeros (x = 0 adds nothing when consumed).  The
    // scalar offset (the super-block's column offset) is outside the hardware
    // range check, so a chunk past the row (ragged d_in) gets the out-of-range
    // lane offset for W_base, its sign byte and x alike.
    auto issue = [&](int b, int t) {
        const bool live = t < nt;
        const int sb = wave + t * KW;
        const uint32_t so = (uint32_t)sb * (kSuperK * 2);
        const uint32_t wv = live ? wrow : kInvalidOffset;
        const uint32_t sv = live ? srow : kInvalidOffset;
        if constexpr (EVEN) {
            const uint4 v = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, sv, (uint32_t)sb * (kSuperK / 8), 0));
            st[b].s[0] = v.x;
            st[b].s[1] = v.y;
            st[b].s[2] = v.z;
            st[b].s[3] = v.w;
        }
#pragma unroll
        for (int jj = 0; jj < JJ; ++jj) {
            bool ok = live;
            if constexpr (!EVEN) {
                ok = ok && (int64_t)sb * (kSuperK / 8) + 4 * jj + q < G;
                st[b].s[jj] = __builtin_amdgcn_raw_buffer_load_b8(rs, ok ? sv + 4 * jj + q : kInvalidOffset,
                                                                  (uint32_t)sb * (kSuperK / 8), 0);
            }
            st[b].w[jj] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, ok ? wv + 64 * jj : kInvalidOffset, so, 0));
            st[b].x[jj] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? xrow + 64 * jj : kInvalidOffset, so, 0));
        }
    };
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    auto compute = [&](int b) {
#pragma unroll
        for (int jj = 0; jj < JJ; ++jj) {
            const uint32_t byte = EVEN ? (st[b].s[jj] >> (8 * q)) & 0xFFu : st[b].s[jj];
            const uint4 e = weff8(sgn, byte, st[b].w[jj], a);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, st[b].x[jj]),
                                                          __builtin_bit_cast(bf16x8, e), acc, 0, 0, 0);
        }
    };
    // Scheduling barriers keep each stage's loads in issue order, so the
    // compiler's wait before a compute leaves the next stage in flight.  The
    // last two computes may consume dead (all-zero x) stages: no branch.
    issue(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    issue(1, 1);
    __builtin_amdgcn_sched_barrier(0);
    for (int t = 0; t + 2 < nt; t += 2) {
        compute(0);
        __builtin_amdgcn_sched_barrier(0);
        issue(0, t + 2);
        __builtin_amdgcn_sched_barrier(0);
        compute(1);
        __builtin_amdgcn_sched_barrier(0);
        issue(1, t + 3);
        __builtin_amdgcn_sched_barrier(0);
    }
    compute(0);
    compute(1);

    red[wave][lane] = acc;
    __syncthreads();
    if (threadIdx.x < 256) {
        // D layout of the 16 x 16 tile: lane l holds tokens 4 (l / 16) + r of row l % 16
        const int src = threadIdx.x >> 2, r = threadIdx.x & 3;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < KW; ++w)
            v += red[w][src][r];
        const int tok = 4 * (src >> 4) + r;
        const int64_t row = n0 + (src & 15);
        if (tok < m && row < R)
            y[(int64_t)tok * ldy + row] = to_bf16(v);
    }
}

// ------------------------------------------------- m in 5..16, whole rows
// gemv_rows (d_in a multiple of 4096): the memory side of gemv_stream at
// m = 1 -- each of the 16 waves of a workgroup streams RW whole rows (rows
// w, w + 16, ...), 1 KB of W_base per load instruction, a ring of D register
// stages of 512 columns -- with the token products on the matrix cores.
// Every wave forms W_eff for its rows (lane l: columns 8l .. 8l + 7 of each
// step) and writes it to an LDS tile of the workgroup's 16 RW rows, NB steps
// at a time; after one barrier wave w reads, for each of those steps and each
// block of 16 rows, the MFMA B operand of its 32-column slice (lane (j, q):
// row j of the block, columns 32w + 8q .. +7) and runs one
// v_mfma_f32_16x16x32_bf16 with A = the same columns of the 16 tokens (L2
// reads, prefetched with the stage, shared by the RW blocks).  16-byte chunk
// c of row j sits at LDS position c ^ (j mod 16), so the tile's writes (one
// row per wave) and the fragment reads (16 rows per read) are both free of
// bank conflicts.  The 16 waves' partial 16 x 16 tiles (disjoint column
// slices) are summed through LDS in wave order.  Three plans:
//  - rows of 4096 (one ring of D = 8 stages holds the row): RW = 1, the
//    whole ring in one barrier group (NB = 8) and one tile buffer.  Measured
//    on 4096 x 4096 at m = 16 (same box): one barrier per step 10.45 us, per
//    2 steps 10.0, per 4 steps 9.75, per 8 steps 9.6 with the rotated step
//    order below (10.0 without it).
//  - longer rows, at least kRowsPairMin of them: RW = 2 (x read once per 32
//    rows instead of 16), D = 4, groups of NB = 2 steps into two tile
//    buffers, so one barrier per group and the other half of the ring's
//    loads in flight while a group is formed and multiplied.  At m = 16 (same
//    box, graph-timed, us): 8192 x 8192 37.4 -> 27.5, 28672 x 8192 119 -> 96,
//    8192 x 28672 114 -> 86.
//  - few rows (512 .. 2048, so at most 128 workgroups of 16) of at least
//    8192 columns: the row's steps are cut into `splits` parts of whole
//    4-stage rings, one workgroup per (row block, part), each writing fp32
//    sums to the workspace; gemv_split_reduce adds the parts in part order
//    (1024 x 8192 at m = 16: 16.2 -> 8.5 us).
constexpr int kRowsWaves = 16;
// Workgroup b walks its rows' steps starting at step rot(b), so the
// workgroups in flight read different columns of x (and of their rows) at
// any moment instead of all the same ones.  Consecutive workgroups land on
// different XCDs (8, round robin).  One ring per row: rot = b mod S.  The
// two-row plan adds b / 8, so the workgroups of one XCD also start apart
// (same box, graph-timed, us: m = 16 8192 x 8192 27.2 -> 25.5, 28672 x 8192
// 97.7 -> 91.4; m = 8 26.7 -> 24.1, 93.7 -> 88.4; 8192 x 28672 unchanged).
// On 4096 x 4096 at m = 16 the same spread costs 9.28 -> 9.52 us.
constexpr int kRowsNB = 8;
// Rows from which the two-row plan still gives every CU a workgroup.
constexpr int64_t kRowsPairMin = 32 * 256;

template <int D, int NB, int RW, int NBUF, bool SPLIT, bool PER_MATRIX>
__global__ __launch_bounds__(64 * kRowsWaves) void gemv_rows(const uint16_t *__restrict__ x, int m,
                                                             const uint16_t *__restrict__ w_base,
                                                             const uint8_t *__restrict__ signs,
                                                             const float *__restrict__ alpha, int64_t R,
                                                             int64_t K, uint16_t *__restrict__ y, int64_t ldy,
                                                             float *__restrict__ partial, int splits)
{
    constexpr int NW = kRowsWaves;
    static_assert(D % NB == 0, "the stage ring holds whole barrier groups");
    static_assert(NBUF == 1 || NBUF == 2, "one tile buffer, or two used in turn");
    __shared__ __attribute__((aligned(16))) float sgn[64];
    // W_eff of NB steps: [buffer][step][row][chunk position]
    __shared__ uint4 tile[NBUF][NB][NW * RW][64];
    fill_sign_table(sgn);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 15, q = lane >> 4;  // fragment lane: row / token j, k-chunk q
    // SPLIT: workgroup b takes row block b mod nblk and the part b / nblk of
    // the row's steps (the host makes every part a whole number of rings)
    const int nblk = SPLIT ? (int)gridDim.x / splits : (int)gridDim.x;
    const int blk = SPLIT ? (int)blockIdx.x % nblk : (int)blockIdx.x;
    const int part = SPLIT ? (int)blockIdx.x / nblk : 0;
    const int64_t n0 = (int64_t)blk * NW * RW;
    const int64_t G = K >> 3;
    const int S = (int)(G >> 6) / (SPLIT ? splits : 1);  // this workgroup's 512-column steps
    const int s_first = part * S;
    const int rot = RW == 1 ? blk % S : (blk + (blk >> 3)) % S;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w_base, R * K * 2);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(signs, R * G);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (int64_t)m * K * 2);
    // rows past R and tokens past m use the out-of-range lane offset (zeros);
    // the scalar offset (the step) stays inside a valid row
    uint32_t wrow[RW], srow[RW];
    float a[RW];
#pragma unroll
    for (int k = 0; k < RW; ++k) {
        const int64_t row = n0 + wave + 16 * k;
        const bool ok = row < R;
        a[k] = PER_MATRIX ? alpha[0] : alpha[ok ? row : R - 1];
        wrow[k] = ok ? (uint32_t)(row * K * 2 + 16 * lane) : kInvalidOffset;
        srow[k] = ok ? (uint32_t)(row * G + lane) : kInvalidOffset;
    }
    const uint32_t xoff = j < m ? (uint32_t)(j * K * 2 + (32 * wave + 8 * q) * 2) : kInvalidOffset;

    uint4 wq[D][RW], xq[D];
    uint32_t sq[D][RW];
    auto load = [&](int d, int s) {
        int c = s + rot;  // the step's columns
        c = (c >= S ? c - S : c) + s_first;
#pragma unroll
        for (int k = 0; k < RW; ++k) {
            wq[d][k] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, wrow[k], (uint32_t)c * 1024u, kStream));
            sq[d][k] = __builtin_amdgcn_raw_buffer_load_b8(rs, srow[k], (uint32_t)c * 64u, kStream);
        }
        xq[d] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff, (uint32_t)c * 1024u, 0));
    };
    f32x4 acc[RW];
#pragma unroll
    for (int k = 0; k < RW; ++k)
        acc[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // steps s .. s + NB - 1 held in stages d .. d + NB - 1: every row's W_eff
    // into the tile, one barrier, then each wave's MFMAs.
    auto group = [&](int d, int s) {
        int buf = 0;
        if constexpr (NBUF == 1) {
            if (s > 0)
                __syncthreads();  // the previous group's reads of the tile are done
        } else {
            // group s / NB takes buffer (s / NB) mod 2, last read by the group
            // before the previous one: every wave finished those reads before
            // it passed the previous group's barrier
            buf = (s / NB) & 1;
        }
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int k = 0; k < RW; ++k)
                tile[buf][i][wave + 16 * k][lane ^ wave] = weff8(sgn, sq[d + i][k], wq[d + i][k], a[k]);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int k = 0; k < RW; ++k) {
                const uint4 b = tile[buf][i][16 * k + j][(4 * wave + q) ^ j];
                acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xq[d + i]),
                                                                 __builtin_bit_cast(bf16x8, b), acc[k], 0, 0, 0);
            }
    };
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load(d, d);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int s0 = 0; s0 < S - D; s0 += D) {
#pragma unroll
        for (int d = 0; d < D; d += NB) {
            group(d, s0 + d);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < NB; ++i)
                load(d + i, s0 + d + i + D);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int d = 0; d < D; d += NB)
        group(d, S - D + d);

    // sum the waves' partial tiles in wave order (the tile holds them:
    // every read of the last group is done after this barrier)
    static_assert(NBUF * NB >= 1, "the tile holds the NW * RW partial tiles");
    __syncthreads();
    f32x4 *red = reinterpret_cast<f32x4 *>(&tile[0][0][0][0]);
#pragma unroll
    for (int k = 0; k < RW; ++k)
        red[(wave * RW + k) * 64 + lane] = acc[k];
    __syncthreads();
    if (threadIdx.x < 256 * RW) {
        // block k = threadIdx / 256; D layout of its 16 x 16 tile: lane l holds
        // tokens 4 (l / 16) + r of row l % 16
        const int k = threadIdx.x >> 8, t = threadIdx.x & 255;
        const int src = t >> 2, r = t & 3;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w)
            v += red[(w * RW + k) * 64 + src][r];
        const int tok = 4 * (src >> 4) + r;
        const int64_t rr = n0 + 16 * k + (src & 15);
        if (tok < m && rr < R) {
            if constexpr (SPLIT)
                partial[((int64_t)part * m + tok) * R + rr] = v;
            else
                y[(int64_t)tok * ldy + rr] = to_bf16(v);
        }
    }
}

// y[t][r] = bf16(sum over the parts, in part order, of partial[part][t][r]).
__global__ __launch_bounds__(256) void gemv_split_reduce(const float *__restrict__ partial, int splits, int m,
                                                         int64_t R, uint16_t *__restrict__ y, int64_t ldy)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)m * R)
        return;
    const int tok = (int)(i / R);
    const int64_t r = i - (int64_t)tok * R;
    const float *src = partial + (int64_t)tok * R + r;
    const int64_t stride = (int64_t)m * R;
    // four parts' loads in flight at a time, added in part order
    float v = 0.0f;
    int p = 0;
    for (; p + 4 <= splits; p += 4) {
        const float a0 = src[p * stride], a1 = src[(p + 1) * stride];
        const float a2 = src[(p + 2) * stride], a3 = src[(p + 3) * stride];
        v += a0;
        v += a1;
        v += a2;
        v += a3;
    }
    for (; p < splits; ++p)
        v += src[p * stride];
    y[(int64_t)tok * ldy + r] = to_bf16(v);
}

// ---------------------------------------------------------------- launch
// Largest D <= dmax that divides S.
int pipeline_depth(int64_t S, int dmax)
{
    int d = dmax;
    while (d > 1 && S % d != 0)
        --d;
    return d;
}

struct Args {
    const uint16_t *x;
    int m;
    const uint16_t *w;
    const uint8_t *sg;
    const float *a;
    bool pm;
    int64_t rows, d_in, ldy;
    uint16_t *y;
    hipStream_t s;
};

// x goes through LDS for MT >= kXLdsMinM tokens and at most kXLdsMax bytes.
constexpr int kXLdsMinM = 2;
// Largest x (m * d_in bf16) the m <= 4 kernels keep in LDS.
constexpr int64_t kXLdsMax = 64 * 1024;

template <int MT, int RW, int D>
hipError_t launch_stream(const Args &g)
{
    const bool even = (g.d_in >> 3) % 64 == 0;
    const int64_t xbytes = (int64_t)g.m * g.d_in * 2;
    constexpr int NW = stream_waves<MT>();
    const dim3 grid((unsigned)((g.rows + NW * RW - 1) / (NW * RW))), block(64 * NW);
#define BD_STREAM(PM, EV, XL, LDS)                                                                          \
    hipLaunchKernelGGL((gemv_stream<MT, RW, D, PM, EV, XL>), grid, block, LDS, g.s, g.x, g.m, g.w, g.sg, g.a, \
                       g.rows, g.d_in, g.y, g.ldy)
    if constexpr (MT >= kXLdsMinM) {
        if (even && xbytes <= kXLdsMax) {
            if (g.pm) BD_STREAM(true, true, true, (unsigned)xbytes);
            else BD_STREAM(false, true, true, (unsigned)xbytes);
            return hipGetLastError();
        }
    }
    if (g.pm) {
        if (even) BD_STREAM(true, true, false, 0);
        else BD_STREAM(true, false, false, 0);
    } else {
        if (even) BD_STREAM(false, true, false, 0);
        else BD_STREAM(false, false, false, 0);
    }
#undef BD_STREAM
    return hipGetLastError();
}

template <int MT, int RW>
hipError_t dispatch_stream(const Args &g, int dmax)
{
    const int64_t S = ((g.d_in >> 3) + 63) >> 6;
    switch (pipeline_depth(S, dmax)) {
    case 8: if constexpr (MT == 1) return launch_stream<MT, RW, 8>(g);
            [[fallthrough]];
    case 7: if constexpr (MT == 1) return launch_stream<MT, RW, 7>(g);
            [[fallthrough]];
    case 6: if constexpr (MT == 1) return launch_stream<MT, RW, 6>(g);
            [[fallthrough]];
    case 5: if constexpr (MT == 1) return launch_stream<MT, RW, 5>(g);
            [[fallthrough]];
    case 4: return launch_stream<MT, RW, 4>(g);
    case 3: return launch_stream<MT, RW, 3>(g);
    case 2: return launch_stream<MT, RW, 2>(g);
    default: return launch_stream<MT, RW, 1>(g);
    }
}

hipError_t launch_mfma(const Args &g)
{
    const bool even = g.d_in % kSuperK == 0;
    const dim3 grid((unsigned)((g.rows + 15) / 16)), block(64 * kMfmaWaves);
#define BD_MFMA(PM, EV)                                                                                     \
    hipLaunchKernelGGL((gemv_mfma<PM, EV>), grid, block, 0, g.s, g.x, g.m, g.w, g.sg, g.a, g.rows, \
                       g.d_in, g.y, g.ldy)
    if (g.pm) {
        if (even) BD_MFMA(true, true);
        else BD_MFMA(true, false);
    } else {
        if (even) BD_MFMA(false, true);
        else BD_MFMA(false, false);
    }
#undef BD_MFMA
    return hipGetLastError();
}

// gemv_rows takes d_in a multiple of 4096: whole rings of 8 stages of 512
// columns (the ring holds whole barrier groups of kRowsNB = 8 steps), or of 4
// stages in the two-row plan.
constexpr int kRowsDepth = 8;
static_assert(kRowsDepth % kRowsNB == 0, "the stage ring holds whole barrier groups");
bool rows_shape(int64_t d_in) { return d_in % (512 * kRowsDepth) == 0; }

hipError_t launch_rows(const Args &g, int splits, float *partial)
{
    const dim3 block(64 * kRowsWaves);
#define BD_ROWS(D, NB, RW, NBUF, SPLIT, NSPLIT)                                                                    \
    do {                                                                                                            \
        const dim3 grid((unsigned)((g.rows + kRowsWaves * RW - 1) / (kRowsWaves * RW) * NSPLIT));                  \
        if (g.pm)                                                                                                   \
            hipLaunchKernelGGL((gemv_rows<D, NB, RW, NBUF, SPLIT, true>), grid, block, 0, g.s, g.x, g.m, g.w, g.sg, \
                               g.a, g.rows, g.d_in, g.y, g.ldy, partial, NSPLIT);                                   \
        else                                                                                                        \
            hipLaunchKernelGGL((gemv_rows<D, NB, RW, NBUF, SPLIT, false>), grid, block, 0, g.s, g.x, g.m, g.w,      \
                               g.sg, g.a, g.rows, g.d_in, g.y, g.ldy, partial, NSPLIT);                             \
    } while (0)
    if (splits > 1) {
        BD_ROWS(4, 4, 1, 1, true, splits);
        const int64_t n = (int64_t)g.m * g.rows;
        hipLaunchKernelGGL(gemv_split_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, g.s, partial, splits,
                           g.m, g.rows, g.y, g.ldy);
    } else if (g.d_in > 512 * kRowsDepth && g.rows >= kRowsPairMin) {
        BD_ROWS(4, 2, 2, 2, false, 1);
    } else {
        BD_ROWS(kRowsDepth, kRowsNB, 1, 1, false, 1);
    }
#undef BD_ROWS
    return hipGetLastError();
}

// Does launch_gemv take the whole-row kernel for this m and width?
bool uses_rows(int m, int64_t d_in)
{
    if (m <= 2 || !rows_shape(d_in))
        return false;
    return m > 4 || (int64_t)m * d_in * 2 > kXLdsMax;
}

}  // namespace

int gemv_splits(int m, int64_t rows, int64_t d_in)
{
    if (m < 1 || m > kGemvMaxM || !uses_rows(m, d_in) || d_in < 8192)
        return 1;
    const int64_t blocks = (rows + kRowsWaves - 1) / kRowsWaves;
    // (and one launch chunk: W_base well below 2 GiB)
    if (rows < 512 || blocks > 128 || rows * d_in * 2 >= ((int64_t)1 << 30))
        return 1;
    // the fewest parts that give about one workgroup per CU, each part a whole
    // number of 4-stage rings
    const int S = (int)(d_in / 512);
    const int target = (int)((256 + blocks - 1) / blocks);
    int best = 1;
    for (int sp = 2; sp <= S / 4; ++sp) {
        if (S % sp != 0 || (S / sp) % 4 != 0)
            continue;
        best = sp;
        if (sp >= target)
            break;
    }
    return best;
}

size_t gemv_workspace_bytes(int m, int64_t rows, int64_t d_in)
{
    const int sp = gemv_splits(m, rows, d_in);
    return sp > 1 ? (size_t)sp * (size_t)m * (size_t)rows * sizeof(float) : 0;
}

// Rows are launched in chunks whose W_base stays below 2 GiB (the kernels
// address it with 32-bit buffer offsets); y keeps its full row stride.  The
// split plan (and its workspace, sized for d_out) only ever applies to a
// matrix launched whole.
hipError_t launch_gemv(const uint16_t *x, int m, const uint16_t *w_base, const uint8_t *signs,
                       const float *alpha, bool per_matrix, int64_t d_out, int64_t d_in,
                       uint16_t *y, void *workspace, hipStream_t s)
{
    const int64_t G = d_in >> 3;
    const int64_t max_rows = std::max<int64_t>(16, (((int64_t)1 << 31) - 1) / (d_in * 2) / 16 * 16);
    const int splits = d_out <= max_rows ? gemv_splits(m, d_out, d_in) : 1;
    if (splits > 1 && workspace == nullptr)
        return hipErrorInvalidValue;
    for (int64_t r0 = 0; r0 < d_out; r0 += max_rows) {
        Args g{x, m, w_base + r0 * d_in, signs + r0 * G, per_matrix ? alpha : alpha + r0, per_matrix,
               std::min(max_rows, d_out - r0), d_in, d_out, y + r0, s};
        hipError_t e;
        if (m <= 1)
            e = dispatch_stream<1, 1>(g, 8);
        else if (m <= 2)
            // one row per wave when x sits in LDS; two when x comes from L2
            // (its reads per weight byte halve)
            e = (G % 64 == 0 && (int64_t)m * g.d_in * 2 <= kXLdsMax) ? dispatch_stream<2, 1>(g, 4)
                                                                     : dispatch_stream<2, 2>(g, 4);
        else if (m <= 4 && !((int64_t)m * g.d_in * 2 > kXLdsMax && rows_shape(g.d_in)))
            e = dispatch_stream<4, 1>(g, 4);  // x in LDS, or a width the whole-row kernel does not take
        else if (rows_shape(g.d_in))
            e = launch_rows(g, splits, static_cast<float *>(workspace));
        else
            e = launch_mfma(g);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace bd

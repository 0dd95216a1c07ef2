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
// Tile: 256 tokens x 256 output features per workgroup (or 128 features in
// the eight-wave kernel when a call has few tiles), K stepped by 64.
// Two kernels share the tiling:
//  - gemm_tiles_w8 (d_in a multiple of 64: every 70B-class shape), eight
//    waves; its own comment below gives the pipeline;
//  - gemm_tiles (any d_in that is a multiple of 8, with a masked K tail),
//    four waves; wave w owns output features [64w, 64w+64) of the tile for
//    all 256 tokens (8 x 2 blocks of v_mfma_f32_32x32x16_bf16, 256 fp32
//    accumulators per lane).  Per K step t: the activation tile of step t+1
//    is copied HBM -> LDS by direct-to-LDS loads (no VGPRs, no LDS write
//    instructions) into the other of two LDS buffers; each wave loads its
//    own 64 x 64 slice of W_base and the sign bytes two steps ahead into
//    VGPRs, in the MFMA B-operand layout (lane l: feature l%32, 8 consecutive
//    k), and while the MFMAs of step t run the VALU forms step t+1's
//    W_eff = bf16(W_base + +-alpha) fragments in VGPRs; one barrier per step.
// In both, activation rows sit in LDS unpadded with the 16-byte chunks of row
// r permuted by c ^ ((r >> 1) & 7), so the 16-byte fragment reads of 32
// consecutive rows spread over all banks; each weight is rebuilt exactly once
// per workgroup and W_eff is never written to HBM; out-of-range loads use
// buffer offsets past the end (they read zero), so no load sits under a
// branch.  Workgroups are remapped so that the ones sharing an
// output-feature tile run on the same XCD (blocks are dealt round-robin over
// the 8 XCDs), so each W_base tile is fetched into one L2 once.
#include <mutex>
#include <type_traits>

#include "bd_device.h"
#include "bd_launch.h"

namespace bd {
namespace {

constexpr int BM = kGemmBM, BN = kGemmBN, BK = 64;
constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int64_t kCus = 256;

__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t nb)
{
    const int64_t per = nb / kXcds;
    if (b >= per * kXcds)
        return b;
    return (b % kXcds) * per + b / kXcds;
}

typedef const __attribute__((address_space(1))) void gbl_void;

struct WRaw {
    uint4 w[2][4];     // [nb][kb]: 8 consecutive bf16 of one feature row
    uint32_t s[2][2];  // [nb]: sign bytes of the 64 columns of the step (8 bytes)
};

// General kernel (d_in a multiple of 8, not of 64): sign rows are not
// 8-byte aligned, so a step's 8 sign bytes are fetched byte by byte.
template <bool PER_MATRIX, bool GATHER>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_tiles(const uint16_t *__restrict__ x, int64_t M, const uint16_t *__restrict__ w_base,
                const uint8_t *__restrict__ signs_all, const float *__restrict__ alpha_all,
                int64_t N, int64_t K, uint16_t *__restrict__ y, int64_t m_tiles,
                const int32_t *__restrict__ table, int32_t n_variants)
{
    __shared__ __attribute__((aligned(16))) uint16_t xs[2 * BM * BK];
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

    const int64_t G = K >> 3;
    const int T = (int)((K + BK - 1) / BK);
    const int hi = lane >> 5;  // which 8-column half of a 16-column k block

    // Buffer resources: 32-bit byte offsets, hardware bounds checks (loads
    // past the end return zero, stores past it are dropped).
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, M * K * 2);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w_base, N * K * 2);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(signs, N * G);

    // ---- activation DMA: wave w copies slots [512w, 512w + 512) of a tile,
    // slot s = 8 * row + p holding logical chunk p ^ ((row >> 1) & 7) of
    // tile row `row`; instruction j covers rows 64w + 8j .. 64w + 8j + 7.
    // Rows past M read zeros; columns past K read the next row (finite, and
    // multiplied by the zero W_eff of those columns).
    uint32_t xoff[GATHER ? 8 : 2];
    int64_t xrow_stride = 0;  // bytes between instruction j and j+1 (dense)
    {
        const int p = lane & 7;
#pragma unroll
        for (int j = 0; j < (GATHER ? 8 : 2); ++j) {
            const int row = wave * 64 + j * 8 + (lane >> 3);
            const int c = p ^ (((j & 1) * 4 + (lane >> 4)) & 7);
            int64_t tok;
            if constexpr (GATHER)
                tok = rows_s[row];
            else
                tok = m0 + row;
            xoff[j] = (tok < 0 || tok >= M) ? kInvalidOffset : (uint32_t)((tok * K + c * 8) * 2);
        }
        xrow_stride = 8 * K * 2;
    }
    auto dma_x = [&](int t, int buf) {
        const uint32_t kbytes = (uint32_t)((int64_t)t * BK * 2);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t vo;
            if constexpr (GATHER)
                vo = xoff[j] + kbytes;
            else
                vo = xoff[j & 1] + (uint32_t)((j >> 1) * 2 * xrow_stride) + kbytes;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(xs + buf * BM * BK + (wave * 8 + j) * 512), 16,
                                                     vo, 0, 0, 0);
        }
    };

    // ---- weights: lane's feature rows and per-row alpha
    uint32_t woff[2], soff[2];
    float a[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int64_t n = n0 + wave * 64 + nb * 32 + (lane & 31);
        const bool ok = n < N;
        woff[nb] = ok ? (uint32_t)((n * K + 8 * hi) * 2) : kInvalidOffset;
        soff[nb] = ok ? (uint32_t)(n * G) : kInvalidOffset;
        a[nb] = PER_MATRIX ? alpha[0] : (ok ? alpha[n] : 0.0f);
    }
    auto load_w = [&](WRaw &r, int t) {
        const uint32_t k0b = (uint32_t)((int64_t)t * BK * 2);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                r.w[nb][kb] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, woff[nb] + k0b + kb * 32, 0, 0));
            uint32_t v[2] = {0, 0};
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i >> 2] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, soff[nb] + (uint32_t)(t * 8) + i, 0, 0)
                             << (8 * (i & 3));
            r.s[nb][0] = v[0];
            r.s[nb][1] = v[1];
        }
    };
    auto build_b = [&](bf16x8 (&B)[2][4], const WRaw &r, int t) {
        const int64_t k0 = (int64_t)t * BK;
        const bool tail = k0 + BK > K;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int byte_i = kb * 2 + hi;  // sign byte of this lane's 8 columns
                const uint32_t byte = (r.s[nb][byte_i >> 2] >> (8 * (byte_i & 3))) & 0xFFu;
                uint4 e = weff_group(r.w[nb][kb], byte, a[nb]);
                if (tail && k0 + kb * 16 + 8 * hi >= K)
                    e = make_uint4(0, 0, 0, 0);
                B[nb][kb] = __builtin_bit_cast(bf16x8, e);
            }
        }
    };

    f32x16 acc[8][2];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[mb][nb][v] = 0.0f;

    // A fragment address within a buffer: row mb*32 + (lane&31), logical
    // chunk kb*2 + hi, stored at chunk position (kb*2 + hi) ^ ((row >> 1) & 7).
    const int arow = lane & 31;
    const int asw = (arow >> 1) & 7;
    auto mfma_step = [&](const bf16x8 (&B)[2][4], int buf) {
        const uint16_t *base = xs + buf * BM * BK + arow * BK;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int chunk = (kb * 2 + hi) ^ asw;
#pragma unroll
            for (int mb = 0; mb < 8; ++mb) {
                const bf16x8 A = *reinterpret_cast<const bf16x8 *>(base + mb * 32 * BK + chunk * 8);
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B[nb][kb], acc[mb][nb], 0, 0, 0);
            }
        }
    };

    // ---- prologue: x(0) -> LDS[0], W(0), W(1); build B(0)
    WRaw wr[2];
    bf16x8 B[2][2][4];
    dma_x(0, 0);
    load_w(wr[0], 0);
    load_w(wr[1], T > 1 ? 1 : 0);
    build_b(B[0], wr[0], 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- main loop, unrolled by two so buffers and register stages are static
    auto step = [&](int t, auto cur_c) {
        constexpr int cur = decltype(cur_c)::value;
        constexpr int nxt = 1 - cur;
        const int t1 = t + 1 < T ? t + 1 : T - 1;
        const int t2 = t + 2 < T ? t + 2 : T - 1;
        dma_x(t1, nxt);              // 8 vector-memory ops
        load_w(wr[cur], t2);         // W(t+2) into the stage W(t) used to occupy
        // keep the loads ahead of the work that follows (the scheduler would
        // otherwise hoist the W_eff build above them and stall on W(t+1))
        __builtin_amdgcn_sched_barrier(0);
        mfma_step(B[cur], cur);
        build_b(B[nxt], wr[nxt], t1);
        __builtin_amdgcn_sched_barrier(0);
        // x(t+1) must have landed; W(t+2) (4 x 16-byte loads per feature
        // block plus its sign loads) may stay in flight
        wait_vmcnt<24>();
        __syncthreads();
    };
    int t = 0;
    for (; t + 1 < T; t += 2) {
        step(t, std::integral_constant<int, 0>{});
        step(t + 1, std::integral_constant<int, 1>{});
    }
    if (t < T)
        step(t, std::integral_constant<int, 0>{});

    // Output: lane l holds feature column l%32 of each 32x32 block; register
    // v holds token row 8*(v/4) + 4*(l/32) + v%4 of the block.  Rows and
    // features that do not exist get an out-of-range offset (store dropped).
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(y, M * N * 2);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int64_t j = n0 + wave * 64 + nb * 32 + (lane & 31);
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int i = mb * 32 + 8 * (v >> 2) + 4 * hi + (v & 3);
                int64_t tok;
                if constexpr (GATHER)
                    tok = rows_s[i];
                else
                    tok = m0 + i < M ? m0 + i : -1;
                const uint32_t off = (tok >= 0 && j < N) ? (uint32_t)((tok * N + j) * 2) : kInvalidOffset;
                __builtin_amdgcn_raw_buffer_store_b16(to_bf16(acc[mb][nb][v]), ry, off, 0, 0);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// LDS tiles of the eight-wave kernel: x 2 x 32 KB, W_eff 2 x 32 KB.
constexpr int kXsBytes = BM * BK * 2;                    // 32768
constexpr int kWsBytes = BN * BK * 2;                    // 32768

// ---------------------------------------------------------------------------
// Eight-wave variant (d_in a multiple of 64): two waves per SIMD, so one
// wave's barrier, copy issue and LDS waits are covered by the other's MFMAs.
// Wave (wm, wn) = (wave / 4, wave % 4) owns output rows wm*128 .. +127 and
// features wn*64 .. +63 of the 256 x 256 tile (4 x 2 MFMA tiles of 32 x 32,
// 128 accumulators, so two waves fit the register file); in a tile 128
// features wide, (wave / 2, wave % 2) owns rows wm*64 .. +63 and features
// wn*64 .. +63 (2 x 2 MFMA tiles).  Per K step of 64:
//  - x tile: direct-to-LDS copies one step ahead, into two LDS buffers;
//  - W_base: each wave loads the 32 (16) feature rows of the tile
//    straight into VGPRs two steps ahead (1 KB per instruction: 8 rows x 128
//    contiguous bytes) with their sign bytes, forms W_eff = bf16(W_base +
//    s alpha) for them once (one fma per weight, sign table in LDS), and
//    writes it to a double-buffered LDS tile in
//    the MFMA B-operand layout; every wave then reads its 64 features from
//    there.  W_eff is built exactly once per workgroup and never leaves LDS.
//  - one barrier per step.
constexpr int kThreads8 = 512;
// Tile width TN (features): 256, or 128 for shapes with few tiles.  Waves
// across the features, 32-row MFMA blocks per wave, 8-row W_base groups per
// wave: TN = 256 -> 2 waves over the tokens x 4 over the features, each 128
// tokens x 64 features, 4 groups; TN = 128 -> 4 x 2 waves of 64 tokens x 64
// features, 2 groups.
template <int TN> constexpr int kW8Wn = TN / 64;
template <int TN> constexpr int kW8Mb = BM / 32 / (8 / kW8Wn<TN>);
template <int TN> constexpr int kW8Groups = TN / 64;

template <bool PER_MATRIX, bool GATHER, bool SPLIT, int TN>
__global__ __launch_bounds__(kThreads8) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_tiles_w8(const uint16_t *__restrict__ x, int64_t M, const uint16_t *__restrict__ w_base,
                   const uint8_t *__restrict__ signs_all, const float *__restrict__ alpha_all,
                   int64_t N, int64_t K, uint16_t *__restrict__ y, int64_t m_tiles,
                   const int32_t *__restrict__ table, int32_t n_variants,
                   int64_t k_split, float *__restrict__ partial, int64_t tile0, int64_t n_fast)
{
    // sign table: its 256-byte alignment makes the compiler place it first,
    // at LDS address 0, so a lookup address is just the masked nibble (after
    // the 128 KB of tiles its base would not fit the 16-bit instruction
    // offset and cost an extra VALU op per lookup)
    __shared__ __attribute__((aligned(256))) float sgn[64];
    // separate objects per buffer: a read of one is then tied only to the
    // copies into that one
    __shared__ __attribute__((aligned(16))) uint8_t XS0[kXsBytes];
    __shared__ __attribute__((aligned(16))) uint8_t XS1[kXsBytes];
    __shared__ __attribute__((aligned(16))) uint8_t WE0[kWsBytes];
    __shared__ __attribute__((aligned(16))) uint8_t WE1[kWsBytes];
    __shared__ int32_t rows_s[GATHER ? BM : 1];
    uint8_t *const XSb[2] = {XS0, XS1};
    uint8_t *const WEb[2] = {WE0, WE1};
    fill_sign_table_h(sgn);
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / kW8Wn<TN>, wn = wave % kW8Wn<TN>;
    const int hi = lane >> 5;
    // this launch covers tiles tile0 .. tile0 + gridDim.x - 1
    const int64_t local = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t b = tile0 + local;
    // tile order: token tiles fastest (each XCD's share holds few feature
    // tiles, so W_base is fetched once and x once per XCD) or, with n_fast =
    // the feature-tile count, feature tiles fastest (x once, W_base once per
    // XCD): the smaller operand is the one fetched by every XCD
    const int64_t mt = n_fast ? b / n_fast : b % m_tiles, nt = n_fast ? b % n_fast : b / m_tiles;
    const int64_t n0 = nt * TN;

    int64_t m0 = mt * BM;
    const uint8_t *signs = signs_all;
    const float *alpha = alpha_all;
    if constexpr (GATHER) {
        const int32_t total = table[0];
        if (mt >= total)
            return;
        const int32_t *perm = table + 4;
        const int32_t *tile_v = perm + M;
        const int32_t *tile_row0 = tile_v + m_tiles;
        const int32_t *tile_rows = tile_row0 + m_tiles;
        const int v = tile_v[mt];
        const int row0 = tile_row0[mt], nrows = tile_rows[mt];
        for (int i = threadIdx.x; i < BM; i += kThreads8)
            rows_s[i] = i < nrows ? perm[row0 + i] : -1;
        __syncthreads();
        if (v >= n_variants) {
            for (int i = 0; i < nrows; ++i) {
                const int64_t tok = rows_s[i];
                for (int64_t j = n0 + threadIdx.x; j < min(N, n0 + TN); j += kThreads8)
                    y[tok * N + j] = 0;
            }
            return;
        }
        signs = signs_all + (int64_t)v * N * (K >> 3);
        alpha = PER_MATRIX ? alpha_all + v : alpha_all + (int64_t)v * N;
        m0 = 0;
    }

    const int64_t G = K >> 3;
    const int64_t k_begin = (int64_t)blockIdx.y * k_split;
    const int T = (int)((min(K, k_begin + k_split) - k_begin) / BK);
    const uint32_t kx0 = (uint32_t)(k_begin * 2);
    const uint32_t ks0 = (uint32_t)(k_begin / 8);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, M * K * 2);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w_base, N * K * 2);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(signs, N * G);

    // x copies: instruction j (0..3) of wave w covers tile rows 32w + 8j ..
    // +7; lane l writes LDS position l & 7 of row 8j + l / 8, which holds
    // logical chunk (l & 7) ^ ((row >> 1) & 7).  Every row has its own lane
    // offset (out of range past M); the scalar offset carries only the K
    // position, which the hardware range check does not cover and which
    // stays inside the row.
    const int p = lane & 7;
    uint32_t xoff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = wave * 32 + j * 8 + (lane >> 3);
        const int c = p ^ (((j & 1) * 4 + (lane >> 4)) & 7);
        int64_t tok;
        if constexpr (GATHER)
            tok = rows_s[row];
        else
            tok = m0 + row;
        xoff[j] = (tok < 0 || tok >= M) ? kInvalidOffset : (uint32_t)((tok * K + c * 8) * 2);
    }
    auto dma_x = [&](int t, int buf) {
        const uint32_t kb = kx0 + (uint32_t)(t * BK * 2);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(XSb[buf] + (wave * 4 + j) * 1024), 16, xoff[j],
                                                     kb, 0, 0);
    };

    // W_base rows of this wave: load i (0 .. NG-1) covers feature rows
    // 8 NG wave + 8i .. +7, lane l -> row 8i + l / 8, chunk l & 7 (8
    // columns).  One lane offset for i = 0; the 8i rows go in the scalar
    // offset, which the hardware range check does not cover.  That is safe
    // because the host runs this kernel only with N a multiple of 32: the
    // wave's 8 NG rows (32 or 16, from a multiple of that) are then all below
    // N or all at or past it, so a valid row nw implies valid rows nw + 8i,
    // and an invalid one has the out-of-range lane offset (zeros).
    constexpr int NG = kW8Groups<TN>, MB = kW8Mb<TN>;
    const int64_t nw = n0 + wave * (8 * NG) + (lane >> 3);
    const uint32_t woff = nw < N ? (uint32_t)((nw * K + p * 8) * 2) : kInvalidOffset;
    const uint32_t soff = nw < N ? (uint32_t)(nw * G + p) : kInvalidOffset;
    const uint32_t wrow8 = (uint32_t)(8 * K * 2), srow8 = (uint32_t)(8 * G);
    float a[NG];
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        const int64_t n = nw + 8 * i;
        a[i] = PER_MATRIX ? alpha[0] : (n < N ? alpha[n] : 0.0f);
    }
    struct WRaw8 {
        uint4 w[NG];
        uint32_t s[NG];
    };
    // group i of the W_base rows (8 rows x 64 columns) and its sign bytes
    auto load_w = [&](WRaw8 &r, int i, int t) {
        const uint32_t kb = kx0 + (uint32_t)(t * BK * 2);
        const uint32_t ksb = ks0 + (uint32_t)(t * 8);
        r.w[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, woff, kb + i * wrow8, 0));
        r.s[i] = __builtin_amdgcn_raw_buffer_load_b8(rs, soff, ksb + i * srow8, 0);
    };
    // W_eff of load i -> LDS row n_local = 8 NG wave + 8i + l/8, position p ^ swizzle
    auto build_store = [&](const WRaw8 &r, int i, int buf) {
        const int nl = wave * (8 * NG) + i * 8 + (lane >> 3);
        const int sw = ((i & 1) * 4 + (lane >> 4)) & 7;  // (nl >> 1) & 7
        const uint4 e = weff8h(sgn, r.s[i], r.w[i], a[i]);
        *reinterpret_cast<uint4 *>(WEb[buf] + nl * 128 + ((p ^ sw) * 16)) = e;
    };

    // Accumulators in AGPRs: the empty asm with an AGPR constraint makes the
    // compiler select the AGPR form of the MFMA (left alone, it keeps them in
    // VGPRs, where the MFMAs and the W_eff builds contend for the same
    // register file and barely overlap).
    f32x16 acc[MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
            for (int v = 0; v < 16; ++v)
                acc[mb][nb][v] = 0.0f;
            asm volatile("" : "+a"(acc[mb][nb]));
        }

    const int frow = lane & 31;
    const int fsw = (frow >> 1) & 7;
    auto read_a = [&](bf16x8 (&A)[MB], int buf, int kb) {
        const uint8_t *base = XSb[buf] + (wm * (32 * MB) + frow) * 128 + (((kb * 2 + hi) ^ fsw) * 16);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            A[mb] = *reinterpret_cast<const bf16x8 *>(base + mb * 32 * 128);
    };
    auto read_b = [&](bf16x8 (&B)[2], int buf, int kb) {
        const uint8_t *base = WEb[buf] + (wn * 64 + frow) * 128 + (((kb * 2 + hi) ^ fsw) * 16);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
            B[nb] = *reinterpret_cast<const bf16x8 *>(base + nb * 32 * 128);
    };

    // ---- prologue: x(0), x(1) copies; W(0) loaded and built into WE0; W(1)
    // loaded; the k-block 0 fragments of step 0 read
    WRaw8 wr;
    dma_x(0, 0);
    dma_x(T > 1 ? 1 : 0, 1);
#pragma unroll
    for (int i = 0; i < NG; ++i)
        load_w(wr, i, 0);
#pragma unroll
    for (int i = 0; i < NG; ++i) {
        build_store(wr, i, 0);
        load_w(wr, i, T > 1 ? 1 : 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    bf16x8 A[2][MB], B[2][2];
    read_a(A[0], 0, 0);
    read_b(B[0], 0, 0);

    // Step t (x(t) in XS cur, W_eff(t) in WE cur, k-block 0 fragments in
    // registers): k-blocks 0..2 read the next k-block's fragments and run
    // their MFMAs; after them the groups of W_eff(t+1) are formed into WE
    // nxt, each group's registers refilled with W(t+2): with four groups, two
    // after k-block 0 and one after each of k-blocks 1 and 2; with two, one
    // after each of k-blocks 0 and 1 (so every build has MFMAs to overlap).  Then, with every read of buffer cur done, the barrier; after
    // it, x(t+2) is copied into XS cur, step t+1's k-block 0 fragments are
    // read, and step t's last 8 MFMAs (k-block 3, from registers) cover that
    // transition.
    auto mfma_kb = [&](int kb) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[kb & 1][mb], B[kb & 1][nb], acc[mb][nb], 0,
                                                                      0, 0);
    };
    auto step = [&](int t, auto cur_c) {
        constexpr int cur = decltype(cur_c)::value;
        constexpr int nxt = 1 - cur;
        const int t2 = t + 2 < T ? t + 2 : T - 1;
#pragma unroll
        for (int kb = 0; kb < 3; ++kb) {
            read_a(A[(kb + 1) & 1], cur, kb + 1);
            read_b(B[(kb + 1) & 1], cur, kb + 1);
            mfma_kb(kb);
            if constexpr (NG == 4) {
                if (kb == 0) {
                    build_store(wr, 0, nxt);
                    load_w(wr, 0, t2);
                }
                build_store(wr, kb + 1, nxt);
                load_w(wr, kb + 1, t2);  // 2 loads
            } else if (kb < NG) {
                build_store(wr, kb, nxt);
                load_w(wr, kb, t2);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // x(t+1) has landed (the 2 NG W loads issued after it may be in
        // flight), W_eff(t+1) is written and this wave's reads of buffer cur
        // are done
        wait_vmcnt_lgkm0<2 * NG>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        dma_x(t2, cur);  // 4 copies: x(t+2)
        __builtin_amdgcn_sched_barrier(0);
        read_a(A[0], nxt, 0);  // past the last step: valid data, unused
        read_b(B[0], nxt, 0);
        mfma_kb(3);
        __builtin_amdgcn_sched_barrier(0);
    };
    int t = 0;
    for (; t + 1 < T; t += 2) {
        step(t, std::integral_constant<int, 0>{});
        step(t + 1, std::integral_constant<int, 1>{});
    }
    if (t < T)
        step(t, std::integral_constant<int, 0>{});
    // the last step's copy of x (unused) must land before the workgroup's LDS
    // is released
    __builtin_amdgcn_s_waitcnt(0);

    if constexpr (SPLIT) {
        // fp32 partials in accumulator order: [split][tile - tile0][wave][mb][nb][quarter][lane][4]
        const int64_t tiles = (int64_t)gridDim.x;
        float *base = partial + (((int64_t)blockIdx.y * tiles + local) * 8 + wave) * (MB * 2 * 4 * 256);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<float4 *>(base + ((mb * 2 + nb) * 4 + q) * 256 + lane * 4) =
                        make_float4(acc[mb][nb][4 * q], acc[mb][nb][4 * q + 1], acc[mb][nb][4 * q + 2],
                                    acc[mb][nb][4 * q + 3]);
    } else {
        const __amdgpu_buffer_rsrc_t ry = make_rsrc(y, M * N * 2);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const int64_t j = n0 + wn * 64 + nb * 32 + (lane & 31);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int i = wm * (32 * MB) + mb * 32 + 8 * (v >> 2) + 4 * hi + (v & 3);
                    int64_t tok;
                    if constexpr (GATHER)
                        tok = rows_s[i];
                    else
                        tok = m0 + i < M ? m0 + i : -1;
                    const uint32_t off = (tok >= 0 && j < N) ? (uint32_t)((tok * N + j) * 2) : kInvalidOffset;
                    __builtin_amdgcn_raw_buffer_store_b16(to_bf16(acc[mb][nb][v]), ry, off, 0, 0);
                }
            }
        }
    }
}

// Sum the split-K partials of gemm_tiles_w8 in split order (fixed, so the
// result is deterministic) and write bf16 y.  One thread per 4 accumulators;
// partial tile i holds output tile tile0 + i.
template <int TN>
__global__ __launch_bounds__(256) void splitk_reduce(const float *__restrict__ partial, int splits, int64_t tiles,
                                                     int64_t tile0, int64_t m_tiles, int64_t M, int64_t N,
                                                     uint16_t *__restrict__ y, int64_t n_fast)
{
    constexpr int MB = kW8Mb<TN>, WN = kW8Wn<TN>;
    constexpr int kChunks = 8 * MB * 2 * 4;  // 256-float chunks per tile: [wave][mb][nb][quarter]
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over tiles * kChunks chunks * 64 lanes
    const int lane = (int)(gid & 63);
    const int64_t chunk = gid >> 6;
    const int q = (int)(chunk & 3), nb = (int)((chunk >> 2) & 1);
    const int mb = (int)((chunk >> 3) % MB);
    const int wave = (int)((chunk >> 3) / MB % 8);
    const int64_t tile = chunk / kChunks;
    if (tile >= tiles)
        return;
    const int64_t stride = tiles * BM * TN;  // floats per split
    const float *src = partial + chunk * 256 + lane * 4;
    float4 s = *reinterpret_cast<const float4 *>(src);
    for (int sp = 1; sp < splits; ++sp) {
        const float4 v = *reinterpret_cast<const float4 *>(src + sp * stride);
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    const int64_t bt = tile0 + tile;
    const int64_t mt = n_fast ? bt / n_fast : bt % m_tiles, nt = n_fast ? bt % n_fast : bt / m_tiles;
    const int64_t j = nt * TN + (wave % WN) * 64 + nb * 32 + (lane & 31);
    const int64_t i0 = mt * BM + (wave / WN) * (32 * MB) + mb * 32 + 8 * q + 4 * (lane >> 5);
    if (j >= N)
        return;
    const float v4[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int r = 0; r < 4; ++r)
        if (i0 + r < M)
            y[(i0 + r) * N + j] = to_bf16(v4[r]);
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
        int lo = 0, hi = nb - 1;  // last bucket with tstart <= ti (a non-empty one)
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tstart[mid] <= ti)
                lo = mid;
            else
                hi = mid - 1;
        }
        const int32_t r0 = seg[lo] + (ti - tstart[lo]) * BM;
        tile_v[ti] = lo;
        tile_row0[ti] = r0;
        tile_rows[ti] = min(BM, seg[lo + 1] - r0);
    }
}

// The general kernel over all m_tiles x n_tiles tiles (d_in not a multiple of
// 64, or d_out not a multiple of 32).
template <bool GATHER>
hipError_t launch_general(const uint16_t *x, int64_t m, const uint16_t *w_base, const uint8_t *signs,
                         const float *alpha, bool per_matrix, int64_t d_out, int64_t d_in, uint16_t *y,
                         int64_t m_tiles, const int32_t *table, int32_t n_variants, hipStream_t s)
{
    const int64_t n_tiles = (d_out + BN - 1) / BN;
    const dim3 grid((unsigned)(m_tiles * n_tiles)), block(kThreads);
    if (per_matrix)
        hipLaunchKernelGGL((gemm_tiles<true, GATHER>), grid, block, 0, s, x, m, w_base, signs, alpha, d_out,
                           d_in, y, m_tiles, table, n_variants);
    else
        hipLaunchKernelGGL((gemm_tiles<false, GATHER>), grid, block, 0, s, x, m, w_base, signs, alpha, d_out,
                           d_in, y, m_tiles, table, n_variants);
    return hipGetLastError();
}

// One launch of gemm_tiles_w8 (tiles TN features wide) over tiles tile0 ..
// tile0 + count - 1, K cut into `splits` ranges (partials into `partial`,
// then summed by splitk_reduce) or unsplit.
template <bool GATHER, int TN>
hipError_t launch_w8(const uint16_t *x, int64_t m, const uint16_t *w_base, const uint8_t *signs,
                     const float *alpha, bool per_matrix, int64_t d_out, int64_t d_in, uint16_t *y,
                     int64_t m_tiles, const int32_t *table, int32_t n_variants, int64_t tile0, int64_t count,
                     int splits, float *partial, hipStream_t s)
{
    // feature tiles fastest when W_base (d_out rows) is smaller than x (m
    // rows): then every XCD fetches all of W_base and its own share of x
    const int64_t n_fast = !GATHER && d_out < m ? (d_out + TN - 1) / TN : 0;
    const int64_t k_split = splits > 1 ? gemm_k_split(d_in, splits) : d_in;
    const int used = (int)((d_in + k_split - 1) / k_split);
    float *part = used > 1 ? partial : nullptr;
    const dim3 grid((unsigned)count, (unsigned)used);
#define BD_W8(PM, SP)                                                                                      \
    hipLaunchKernelGGL((gemm_tiles_w8<PM, GATHER, SP, TN>), grid, dim3(kThreads8), 0, s, x, m, w_base, signs,   \
                       alpha, d_out, d_in, y, m_tiles, table, n_variants, k_split, part, tile0, n_fast)
    if constexpr (GATHER) {  // the grouped GEMM never splits K
        if (per_matrix) BD_W8(true, false);
        else BD_W8(false, false);
    } else if (per_matrix) {
        if (part) BD_W8(true, true);
        else BD_W8(true, false);
    } else {
        if (part) BD_W8(false, true);
        else BD_W8(false, false);
    }
#undef BD_W8
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || GATHER || part == nullptr)
        return e;
    const int64_t threads = count * (8 * kW8Mb<TN> * 2 * 4) * 64;
    hipLaunchKernelGGL(splitk_reduce<TN>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, part, used,
                       count, tile0, m_tiles, m, d_out, y, n_fast);
    return hipGetLastError();
}

}  // namespace

// How a dense prefill call is cut over the 256 CUs (one 256 x 256 tile per
// CU at a time):
//  - few tiles (under 192): the K loop of every tile is cut into equal
//    64-aligned ranges so the grid covers the CUs; each range keeps at least
//    512 columns (8 steps) to amortise the pipeline fill.  With at most 128
//    such tiles, tiles 128 features wide where that pays (twice as many, so
//    half the K ranges and half the partials to sum for the same grid);
//  - more tiles than CUs with a last partial wave of at most half the CUs:
//    that wave's tiles run as a second launch with K cut in 2 (or 4, 8) so
//    it fills the chip and ends sooner, when every range keeps at least 2048
//    columns (the fixed cost of summing the partials is then repaid);
//  - otherwise one unsplit launch.
// Shapes the eight-wave kernel takes (whole 64-column steps; whole 32-row
// blocks of W_base, see the kernel's W_base loads); the rest run on the
// general kernel.
static bool w8_shape(int64_t d_out, int64_t d_in) { return d_in % 64 == 0 && d_out % 32 == 0; }

GemmPlan gemm_plan(int64_t m, int64_t d_out, int64_t d_in)
{
    GemmPlan p{1, 0, 1, BN};
    if (!w8_shape(d_out, d_in))
        return p;
    const int64_t m_tiles = (m + BM - 1) / BM;
    const int64_t tiles = m_tiles * ((d_out + BN - 1) / BN);
    if (tiles < 192) {
        // K ranges of one launch over `t` tiles
        auto ranges = [&](int64_t t) {
            int sp = 1;
            while (sp < 16 && t * sp < kCus && d_in / (2 * sp) >= 512)
                sp *= 2;
            const int64_t ks = gemm_k_split(d_in, sp);
            return (int)((d_in + ks - 1) / ks);
        };
        p.splits = ranges(tiles);
        // Narrow tiles cost more per flop (half the MFMAs per copied x tile
        // and per fragment read) but need half the K ranges: worth it where
        // the wide plan's ranges are short (at most 1024 columns, where
        // pipeline fill and the partials dominate) or where narrow tiles
        // need no split at all.  Measured: +5-16% on such shapes; -18% on
        // 512 x 8192 x 28672, whose wide ranges are 7168 columns.
        if (tiles <= 128) {
            const int64_t narrow = m_tiles * ((d_out + kGemmBNNarrow - 1) / kGemmBNNarrow);
            const int sp_n = ranges(narrow);
            if (sp_n == 1 || gemm_k_split(d_in, p.splits) <= 1024) {
                p.tn = kGemmBNNarrow;
                p.splits = sp_n;
            }
        }
        return p;
    }
    const int64_t rem = tiles % kCus;
    if (tiles > kCus && rem > 0 && 2 * rem <= kCus) {
        int sp = 1;
        while (sp < 8 && rem * 2 * sp <= kCus && d_in / (2 * sp) >= 2048)
            sp *= 2;
        if (sp > 1) {
            p.tail = rem;
            p.tail_splits = sp;
        }
    }
    return p;
}

int64_t gemm_k_split(int64_t d_in, int splits)
{
    return ((d_in + splits - 1) / splits + BK - 1) / BK * BK;
}

size_t gemm_workspace_bytes(int64_t m, int64_t d_out, int64_t d_in)
{
    const GemmPlan p = gemm_plan(m, d_out, d_in);
    const size_t tile = (size_t)BM * p.tn * sizeof(float);
    if (p.tail > 0)
        return (size_t)p.tail_splits * (size_t)p.tail * tile;
    if (p.splits <= 1)
        return 0;
    const int64_t tiles = ((m + BM - 1) / BM) * ((d_out + p.tn - 1) / p.tn);
    return (size_t)p.splits * (size_t)tiles * tile;
}

hipError_t launch_gemm(const uint16_t *x, int64_t m, const uint16_t *w_base, const uint8_t *signs,
                       const float *alpha, bool per_matrix, int64_t d_out, int64_t d_in,
                       uint16_t *y, void *workspace, hipStream_t s)
{
    const int64_t m_tiles = (m + BM - 1) / BM;
    if (!w8_shape(d_out, d_in))
        return launch_general<false>(x, m, w_base, signs, alpha, per_matrix, d_out, d_in, y, m_tiles, nullptr,
                                           0, s);
    const GemmPlan p = gemm_plan(m, d_out, d_in);
    float *part = static_cast<float *>(workspace);
    if (p.tn == kGemmBNNarrow)
        return launch_w8<false, kGemmBNNarrow>(x, m, w_base, signs, alpha, per_matrix, d_out, d_in, y, m_tiles,
                                               nullptr, 0, 0, m_tiles * ((d_out + p.tn - 1) / p.tn), p.splits,
                                               part, s);
    const int64_t tiles = m_tiles * ((d_out + BN - 1) / BN);
    if (p.tail == 0)
        return launch_w8<false, BN>(x, m, w_base, signs, alpha, per_matrix, d_out, d_in, y, m_tiles, nullptr, 0, 0,
                                    tiles, p.splits, part, s);
    const hipError_t e = launch_w8<false, BN>(x, m, w_base, signs, alpha, per_matrix, d_out, d_in, y, m_tiles,
                                              nullptr, 0, 0, tiles - p.tail, 1, nullptr, s);
    if (e != hipSuccess)
        return e;
    return launch_w8<false, BN>(x, m, w_base, signs, alpha, per_matrix, d_out, d_in, y, m_tiles, nullptr, 0,
                                tiles - p.tail, p.tail, p.tail_splits, part, s);
}

int64_t grouped_max_tiles(int64_t m, int32_t n_variants)
{
    return (m + BM - 1) / BM + (int64_t)n_variants + 1;
}

size_t grouped_workspace_bytes(int64_t m, int32_t n_variants)
{
    return sizeof(int32_t) * (size_t)(4 + m + 3 * grouped_max_tiles(m, n_variants));
}

// ---------------------------------------------------------------------------
// The bucketing table of bitdelta_linear_grouped_noalloc: a device-resident
// array (each GPU holds its own copy until the process ends), sized for the
// largest call that entry point accepts.  bucket_tokens writes every word the
// grouped GEMM reads (the header, the permutation, the tile table), so
// nothing in it needs clearing between calls.
namespace {

constexpr size_t kScratchWords =
    (4 + kGroupedNoallocMaxTokens + 3 * ((kGroupedNoallocMaxTokens + BM - 1) / BM + kMaxVariants + 1) + 63) / 64 * 64;
static __device__ __align__(256) int32_t scratch[kScratchWords];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t *g_scratch[kMaxDevices] = {};

}  // namespace

size_t grouped_scratch_bytes() { return sizeof(int32_t) * kScratchWords; }

hipError_t grouped_scratch(int32_t **table)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
        // once per device, with that device current: the address of this
        // GPU's copy of the array (the array's name in host code is only a
        // host-side stand-in)
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        g_scratch[dev] = static_cast<int32_t *>(p);
    }
    *table = g_scratch[dev];
    return hipSuccess;
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
    if (!w8_shape(d_out, d_in))
        return launch_general<true>(x, m, w_base, signs, alpha, per_matrix, d_out, d_in, y, T, workspace,
                                          n_variants, s);
    return launch_w8<true, BN>(x, m, w_base, signs, alpha, per_matrix, d_out, d_in, y, T, workspace, n_variants, 0,
                           T * ((d_out + BN - 1) / BN), 1, nullptr, s);
}

}  // namespace bd

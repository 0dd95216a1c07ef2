// Device-side helpers shared by the gfx950 kernels of this library.
//
// bf16 values are carried as raw 16-bit patterns packed two per 32-bit word
// (element 2p in the low half, 2p+1 in the high half), which is how a
// row-major bf16 row looks when loaded as dwords.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bd {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Exact widening of the low / high bf16 of a packed pair to fp32.
__device__ __forceinline__ float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round two fp32 values to bf16, nearest-even, packed (lo, hi).  Lowers to one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16(float f) { return (uint16_t)(pack_bf16x2(f, 0.0f) & 0xFFFFu); }

// +alpha where bit i of `bits` is 1, -alpha where it is 0 (alpha's own sign
// bit is flipped by the complement of the delta bit).
__device__ __forceinline__ float signed_alpha(uint32_t bits, int i, float a)
{
    return __uint_as_float(__float_as_uint(a) ^ (((~bits >> i) & 1u) << 31));
}

// W_eff for the two bf16 weights packed in `w`, whose delta bits are bits i
// and i+1 of `bits`: fp32 add, then one rounding to bf16 each.
__device__ __forceinline__ uint32_t weff_pair(uint32_t w, uint32_t bits, int i, float a)
{
    float e0 = lo_f32(w) + signed_alpha(bits, i, a);
    float e1 = hi_f32(w) + signed_alpha(bits, i + 1, a);
    return pack_bf16x2(e0, e1);
}

// W_eff for 8 consecutive weights (one 16-byte load) and their sign byte.
__device__ __forceinline__ uint4 weff_group(uint4 w, uint32_t byte, float a)
{
    uint4 r;
    r.x = weff_pair(w.x, byte, 0, a);
    r.y = weff_pair(w.y, byte, 2, a);
    r.z = weff_pair(w.z, byte, 4, a);
    r.w = weff_pair(w.w, byte, 6, a);
    return r;
}

// sum_k lo/hi products of two packed bf16 pairs, accumulated in fp32.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// Sign table for weff8: entry e holds (bit b of e) ? +1 : -1 for b = 0..3
// (64 floats in LDS, filled by the first 64 threads of the workgroup).
__device__ __forceinline__ void fill_sign_table(float *sgn)
{
    if (threadIdx.x < 64)
        sgn[threadIdx.x] = ((threadIdx.x >> 2) >> (threadIdx.x & 3)) & 1 ? 1.0f : -1.0f;
}

// W_eff for the 8 weights of `w` with sign byte `b` (bit i = weight i): one
// fma per weight with s = +-1 from the table (s * alpha is exact, so the fma
// rounds once, exactly as fp32 W + (+-alpha) does), one v_cvt_pk_bf16_f32 per
// pair.  Same result as weff_group.
__device__ __forceinline__ uint4 weff8(const float *sgn, uint32_t b, uint4 w, float a)
{
    const f32x4 lo = *reinterpret_cast<const f32x4 *>(&sgn[(b & 15u) * 4]);
    const f32x4 hi = *reinterpret_cast<const f32x4 *>(&sgn[((b >> 4) & 15u) * 4]);
    uint4 e;
    e.x = pack_bf16x2(fmaf(lo[0], a, lo_f32(w.x)), fmaf(lo[1], a, hi_f32(w.x)));
    e.y = pack_bf16x2(fmaf(lo[2], a, lo_f32(w.y)), fmaf(lo[3], a, hi_f32(w.y)));
    e.z = pack_bf16x2(fmaf(hi[0], a, lo_f32(w.z)), fmaf(hi[1], a, hi_f32(w.z)));
    e.w = pack_bf16x2(fmaf(hi[2], a, lo_f32(w.w)), fmaf(hi[3], a, hi_f32(w.w)));
    return e;
}

// fp16 form of the sign table, in the same 256 bytes: entry e sits at byte
// 16e and holds (bit b of e) ? +1 : -1 as fp16 for b = 0..3 in its first 8
// bytes (the other 8 are unused).  A lookup is then an 8-byte LDS read
// instead of 16, at the same address as in the fp32 table.
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void fill_sign_table_h(float *sgn)
{
    if (threadIdx.x < 64) {
        const int e = threadIdx.x >> 2, b = threadIdx.x & 3;
        if (b < 2) {
            // two fp16 entries per thread-pair's dword: bits 2b, 2b+1 of e
            const uint32_t lo = ((e >> (2 * b)) & 1) ? 0x3C00u : 0xBC00u;
            const uint32_t hi = ((e >> (2 * b + 1)) & 1) ? 0x3C00u : 0xBC00u;
            reinterpret_cast<uint32_t *>(sgn)[4 * e + b] = lo | (hi << 16);
        }
    }
}

// weff8 with the fp16 table: the fp16 +-1 feeds the fma directly (one
// v_fma_mix_f32 per weight, the conversion of +-1 exact), so the result is the
// same single rounding of f32(W) + s alpha.
__device__ __forceinline__ uint4 weff8h(const float *sgn, uint32_t b, uint4 w, float a)
{
    const uint8_t *t = reinterpret_cast<const uint8_t *>(sgn);
    const f16x4 lo = *reinterpret_cast<const f16x4 *>(t + (b & 15u) * 16);
    const f16x4 hi = *reinterpret_cast<const f16x4 *>(t + (b & 0xF0u));
    uint4 e;
    e.x = pack_bf16x2(fmaf((float)lo[0], a, lo_f32(w.x)), fmaf((float)lo[1], a, hi_f32(w.x)));
    e.y = pack_bf16x2(fmaf((float)lo[2], a, lo_f32(w.y)), fmaf((float)lo[3], a, hi_f32(w.y)));
    e.z = pack_bf16x2(fmaf((float)hi[0], a, lo_f32(w.z)), fmaf((float)hi[1], a, hi_f32(w.z)));
    e.w = pack_bf16x2(fmaf((float)hi[2], a, lo_f32(w.w)), fmaf((float)hi[3], a, hi_f32(w.w)));
    return e;
}

// Streaming (nontemporal) 16-byte global load / store and byte load: data
// touched once, kept out of the way of the caches.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream16(const void *p)
{
    const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld_stream8(const uint8_t *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_stream16(void *p, uint4 v)
{
    __builtin_nontemporal_store((u32x4){v.x, v.y, v.z, v.w}, static_cast<u32x4 *>(p));
}

typedef __attribute__((address_space(3))) void lds_void;

// Lane (VGPR) offset of a row that does not exist: beyond every tensor (all
// tensors a kernel addresses through a buffer resource are below 2 GiB,
// checked on the host), so loads return zero and stores are dropped.
//
// The hardware range check of a raw buffer access covers the lane offset
// (plus the instruction's immediate offset) only; the scalar (SGPR) offset
// is added to the address after the check.  Every kernel here therefore puts
// in the scalar offset only a displacement that stays inside memory the lane
// offset has already validated (a column position inside a valid row), and
// gives each row, chunk or token that may not exist its own lane offset.
constexpr uint32_t kInvalidOffset = 0x80000000u;

// Cache policy of a buffer load that streams data read once (nt).
constexpr int kStream = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    // raw buffer: stride 0, num_records in bytes, default data format word
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // s_waitcnt encoding on gfx9: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// vmcnt(N) and lgkmcnt(0) in one wait.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

}  // namespace bd

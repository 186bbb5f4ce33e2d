// Device-side building blocks shared by the gfx950 kernels: I/O element
// types, buffer resources, and the per-point coefficient step of the binary32
// operation sequence fixed in include/dcnv4.h.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "dcnv4.h"

#pragma clang fp contract(off)

namespace dcnv4 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Buffer-resource word 3 for gfx950 raw (untyped, stride 0) buffers: 32-bit
// data format so that out-of-range dwords read as zero.
constexpr int kRsrcFlags = 0x00020000;
// A byte offset that is out of range for every resource the kernels build
// (every resource covers < 2^31 bytes): reads return zeros.
constexpr uint32_t kOobOffset = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcFlags);
}

// Workgroups are dealt to the 8 XCDs round-robin, each XCD with its own L2.
// A grid of 8 * per_xcd workgroups renumbered so that XCD x runs the
// contiguous logical range [x * per_xcd, (x + 1) * per_xcd): neighbouring
// tiles share an L2.  Decodes workgroup b; false for the padding workgroups
// that round the grid up to a multiple of 8.
__device__ __forceinline__ bool logical_block(uint32_t b, uint32_t total, uint32_t per_xcd, uint32_t* out)
{
    const uint32_t xcd = b & 7u, k = b >> 3;
    const uint32_t l = xcd * per_xcd + k;
    *out = l;
    return k < per_xcd && l < total;
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
}

// ---------------------------------------------------------------------------
// I/O element types.  to_f widens exactly; from_f rounds to nearest even.
// ---------------------------------------------------------------------------

template <int DT> struct Elem;

template <> struct Elem<DCNV4_F32> {
    using S = float;
    static constexpr int kBytes = 4;
    static __device__ __forceinline__ float to_f(S v) { return v; }
    static __device__ __forceinline__ S from_f(float f) { return f; }
    static __device__ __forceinline__ float raw_to_f(uint32_t r) { return __uint_as_float(r); }
};

template <> struct Elem<DCNV4_F16> {
    using S = _Float16;
    static constexpr int kBytes = 2;
    static __device__ __forceinline__ float to_f(S v) { return (float)v; }
    static __device__ __forceinline__ S from_f(float f) { return (S)f; }
    static __device__ __forceinline__ float raw_to_f(uint32_t r) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)r);
    }
};

template <> struct Elem<DCNV4_BF16> {
    using S = uint16_t;
    static constexpr int kBytes = 2;
    static __device__ __forceinline__ float to_f(S v) { return __uint_as_float((uint32_t)v << 16); }
    static __device__ __forceinline__ S from_f(float f) {
        uint32_t u = __float_as_uint(f);
        if ((u & 0x7fffffffu) > 0x7f800000u) return (S)((u >> 16) | 0x40u);   // quiet NaN
        u += 0x7fffu + ((u >> 16) & 1u);
        return (S)(u >> 16);
    }
    static __device__ __forceinline__ float raw_to_f(uint32_t r) { return __uint_as_float(r << 16); }
};

// The two bfloat16 halves of a dword widened to binary32 (exact), one
// v_perm_b32 each.  The byte permute is opaque to the optimiser, so the
// widening stays next to its multiply-add instead of being hoisted to the
// load (which would double the registers the loaded data occupies).
__device__ __forceinline__ float bf16_lo(uint32_t d)
{
    return __uint_as_float(__builtin_amdgcn_perm(d, 0u, 0x05040c0cu));   // d << 16
}
__device__ __forceinline__ float bf16_hi(uint32_t d)
{
    return __uint_as_float(__builtin_amdgcn_perm(d, 0u, 0x07060c0cu));   // d & 0xffff0000
}

// acc[0..E) += w * (the E elements packed in one 16-byte vector), in element
// order, one fmaf per element (fp16 folds the widening into the fma).
template <int DT>
__device__ __forceinline__ void fma_vec16(float* acc, float w, u32x4 v)
{
    if constexpr (DT == DCNV4_F32) {
        acc[0] = fmaf(w, __uint_as_float(v.x), acc[0]);
        acc[1] = fmaf(w, __uint_as_float(v.y), acc[1]);
        acc[2] = fmaf(w, __uint_as_float(v.z), acc[2]);
        acc[3] = fmaf(w, __uint_as_float(v.w), acc[3]);
    } else if constexpr (DT == DCNV4_F16) {
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f16x2 h = __builtin_bit_cast(f16x2, d[i]);
            acc[2 * i] = fmaf(w, (float)h.x, acc[2 * i]);
            acc[2 * i + 1] = fmaf(w, (float)h.y, acc[2 * i + 1]);
        }
    } else {
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = fmaf(w, bf16_lo(d[i]), acc[2 * i]);
            acc[2 * i + 1] = fmaf(w, bf16_hi(d[i]), acc[2 * i + 1]);
        }
    }
}

// Elements per 16-byte vector.
template <int DT> constexpr int kPerVec = 16 / Elem<DT>::kBytes;

// The final binary32 accumulator, made opaque to the optimiser.  Without it
// the compiler may fuse the last fmaf with the narrowing conversion
// (v_fma_mixlo_f16): that rounds once, from the exact value, instead of
// rounding to binary32 first and then to the I/O type, and differs in rare
// ties.  The asm emits no instruction.
__device__ __forceinline__ float settle(float v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// Pack E = kPerVec<DT> accumulators into one 16-byte vector of the I/O type.
template <int DT>
__device__ __forceinline__ u32x4 pack_vec16(const float* acc_in)
{
    using E = Elem<DT>;
    float acc[kPerVec<DT>];
#pragma unroll
    for (int i = 0; i < kPerVec<DT>; ++i) acc[i] = settle(acc_in[i]);
    u32x4 r;
    if constexpr (DT == DCNV4_F32) {
        r.x = __float_as_uint(acc[0]); r.y = __float_as_uint(acc[1]);
        r.z = __float_as_uint(acc[2]); r.w = __float_as_uint(acc[3]);
    } else {
        uint32_t d[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = __builtin_bit_cast(uint16_t, E::from_f(acc[2 * i]));
            const uint32_t hi = __builtin_bit_cast(uint16_t, E::from_f(acc[2 * i + 1]));
            d[i] = lo | (hi << 16);
        }
        r.x = d[0]; r.y = d[1]; r.z = d[2]; r.w = d[3];
    }
    return r;
}

// ---------------------------------------------------------------------------
// Rows of offsets / weights / channels read with buffer loads.
// ---------------------------------------------------------------------------

// Load ND consecutive dwords at a 4-byte aligned byte offset: b128 pieces,
// and the LAST dword always on its own.  Callers may ask for one dword past
// the data they need (a row that starts 2 bytes into a dword); keeping that
// dword in a load of its own means no multi-dword load ever straddles the end
// of a buffer resource, so out-of-range handling only ever zeroes whole
// unneeded loads.
template <int ND>
__device__ __forceinline__ void load_dwords(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t* d)
{
    constexpr int NB = ND - 1;        // dwords before the last
#pragma unroll
    for (int i = 0; i + 4 <= NB; i += 4) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(voff + 4 * i), 0, 0);
        d[i] = v.x; d[i + 1] = v.y; d[i + 2] = v.z; d[i + 3] = v.w;
    }
    d[ND - 1] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(voff + 4 * (ND - 1)), 0, 0);
    constexpr int rem = NB % 4, b = NB - NB % 4;
    if constexpr (rem == 1) {
        d[b] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(voff + 4 * b), 0, 0);
    } else if constexpr (rem == 2) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)(voff + 4 * b), 0, 0);
        d[b] = v.x; d[b + 1] = v.y;
    } else if constexpr (rem == 3) {
        typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
        const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, (int)(voff + 4 * b), 0, 0);
        d[b] = v.x; d[b + 1] = v.y; d[b + 2] = v.z;
    }
}

// NE elements of the I/O type starting at byte offset `start` (aligned to the
// element size), as raw 32-bit containers: element e of a 16-bit type sits in
// the low (e even) or high (e odd) half of word e/2; a 32-bit type in word e.
// Two steps, so that a row can be requested one unit ahead without waiting
// for it: issue() starts the loads, finish() (after the data is needed, one
// pass later) moves a 16-bit row that starts 2 bytes into a dword into place.
template <int DT, int NE>
struct RowLoad {
    static constexpr bool k32 = Elem<DT>::kBytes == 4;
    static constexpr int kWords = k32 ? NE : (NE + 1) / 2;
    // dwords loaded (16-bit types: enough to cover a 2-byte misalignment)
    static constexpr int kLoadDwords = k32 ? NE : (2 * NE + 2 + 3) / 4;
    uint32_t w[kWords];
    uint32_t raw[k32 ? 1 : kLoadDwords];
    uint32_t sh;

    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, uint32_t start)
    {
        if constexpr (k32) {
            load_dwords<NE>(r, start, w);
        } else {
            load_dwords<kLoadDwords>(r, start & ~3u, raw);
            sh = (start & 2u) * 8u;                       // 0 or 16 bits
        }
    }

    __device__ __forceinline__ void finish()
    {
        if constexpr (!k32) {
#pragma unroll
            for (int i = 0; i < kWords; ++i)
                w[i] = __builtin_amdgcn_alignbit(i + 1 < kLoadDwords ? raw[i + 1] : 0u, raw[i], sh);
        }
    }

    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t start)
    {
        issue(r, start);
        finish();
    }

    __device__ __forceinline__ float get(int e) const
    {
        if constexpr (DT == DCNV4_F32) {
            return __uint_as_float(w[e]);
        } else if constexpr (DT == DCNV4_F16) {
            const f16x2 h = __builtin_bit_cast(f16x2, w[e / 2]);
            return (e & 1) ? (float)h.y : (float)h.x;
        } else {
            return (e & 1) ? bf16_hi(w[e / 2]) : bf16_lo(w[e / 2]);
        }
    }
};

// ---------------------------------------------------------------------------
// One sampling point: position, range test, bilinear weights with the dynamic
// weight folded in, exactly in the order fixed by the ABI.  A point outside
// (-1,H) x (-1,W) (or with a NaN coordinate) comes back invalid with all four
// weights +0 and x0 = y0 = 0, so that it can be routed to zeros.
// ---------------------------------------------------------------------------

struct PointCoef {
    float w00, w01, w10, w11;
    int x0, y0;
    bool valid;
};

__device__ __forceinline__ PointCoef point_coef(float dx, float dy, float m, float scale,
                                                float basex, float basey, float fW, float fH)
{
    PointCoef c;
    float px = fmaf(dx, scale, basex);
    float py = fmaf(dy, scale, basey);
    // bitwise & (not &&): no short-circuit, so no branch per point
    c.valid = (px > -1.0f) & (px < fW) & (py > -1.0f) & (py < fH);
    px = c.valid ? px : 0.0f;
    py = c.valid ? py : 0.0f;
    m = c.valid ? m : 0.0f;
    const float fx = floorf(px), fy = floorf(py);
    c.x0 = (int)fx;
    c.y0 = (int)fy;
    const float lx = px - fx, ly = py - fy;
    const float hx = 1.0f - lx, hy = 1.0f - ly;
    const float mhy = m * hy, mly = m * ly;
    c.w00 = mhy * hx;
    c.w01 = mhy * lx;
    c.w10 = mly * hx;
    c.w11 = mly * lx;
    return c;
}

}  // namespace dcnv4

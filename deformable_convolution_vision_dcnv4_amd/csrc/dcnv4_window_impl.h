// DCNv4 forward, "window" kernel family: corner gathers served from LDS.
// The kernel template and its launchers; dcnv4_window.hip instantiates the
// DCNv4 aggregation (raw weights), dcnv4_window_sm.hip the DCNv3-style one
// (softmax-normalised weights, SM), in separate translation units so that
// they compile in parallel.
//
// Operation: jsqmd.com/news/933833 ("不只是卷积的平替：我把DCNv4塞进Stable
// Diffusion的U-Net里"), section 1, code example "DCNv4核心计算流程示例"; the raw,
// signed dynamic weights of the same section's first optimisation and of
// bqwf.cn/news/1148139 section 2.1.  Prior art kept from the pages' kernel
// (jsqmd.com/news/933833 section 1 list; bqwf.cn/news/1148139 section 2.2):
// one pass fuses sampling, interpolation and aggregation; the group's channels
// are handled together so each point's bilinear weights are computed once;
// 16-byte vector accesses.
//
// Why LDS: every output (pixel, group) reads 4 corners x K*K points of Cg
// channels, 36x the bytes of x, at data-dependent addresses.  On gfx950 random
// 16-byte reads from LDS run several times faster than random global reads
// that hit L1 or L2, so each workgroup first copies a window of x (its output
// tile's footprint plus a margin for the offsets) into LDS with coalesced
// 16-byte loads, then gathers from LDS.  A point whose corners leave the
// window (a large offset) is read from global memory instead; a window that
// covers the whole zero-bordered image, [-1,H] x [-1,W], never needs that.
//
// Work layout: one workgroup = (image n, GB consecutive groups, TH x TW
// output tile); one lane = one (pixel, group) unit with all Cg channels, so a
// point's position and weights are computed once and used for all channels.
// LDS layout: one plane per (group, 16-byte channel chunk), rows of `pitch`
// 16-byte entries (pitch a multiple of 16 entries, at least two zero columns
// right of the window).  Lanes of a wave take consecutive output columns, so
// the corners they read sit in consecutive entries of one plane: distinct
// LDS banks except where the offsets scramble them.
// Workgroups are renumbered so that each XCD (workgroups are dealt to the 8
// XCDs round-robin) receives a contiguous run of tiles: neighbouring tiles
// and the groups of one tile share that XCD's L2.

#pragma once

#include <type_traits>

#include "dcnv4_device.h"
#include "dcnv4_kernels.h"

namespace dcnv4 {
namespace {

// Offset rows of a wave's 64 consecutive units, moved through LDS.  Per-lane
// row loads touch 64 different cache lines per instruction (each unit's row
// is a short piece of a pixel's row of all groups), which the texture path
// serves several times slower than loads whose lanes walk memory in order.
// Here piece q = k*64 + lane (k < ND) is dword q % ND of unit q / ND: the
// lanes of one load cover whole rows dword by dword, and the load unit writes
// each dword straight to LDS at position q (no registers held while in
// flight), so unit u's row lands at dwords [u*ND, u*ND + ND) of the wave's
// buffer, from where its lane reads it back.  `rows` holds `rows_bytes`
// bytes of rows (one image's); `base` = byte offset of the first unit's row
// there; consecutive units' rows are `row_bytes` apart.  Rows past the end
// (or a base past it) read as zeros.
template <int ND>
__device__ __forceinline__ void stage_offset_rows(const char* rows, uint32_t rows_bytes, uint32_t* wbuf,
                                                  uint32_t lane, uint32_t base, uint32_t row_bytes)
{
    // the same for every lane of the wave, and folded into the resource's
    // base address: the range check covers the per-lane offsets only
    base = __builtin_amdgcn_readfirstlane(base);
    const uint32_t left = __builtin_amdgcn_readfirstlane(base < rows_bytes ? rows_bytes - base : 0u);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(rows + base, left);
    // recomputed at each call (a few integer operations per load) instead of
    // keeping ND loop-invariant offsets in registers across the whole loop
    asm volatile("" : "+v"(lane));
    // (u, d) of piece lane, then stepped by 64 pieces per load
    uint32_t u = lane / (uint32_t)ND, d = lane - u * (uint32_t)ND;
    constexpr uint32_t du = 64u / ND, dd = 64u % ND;
#pragma unroll
    for (int k = 0; k < ND; ++k) {
        // u < 64 and a row is < 2^24 bytes (the caller checks): 24-bit multiply
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ro, (__attribute__((address_space(3))) void*)(wbuf + k * 64),
                                                 4, (int)(__umul24(u, row_bytes) + 4u * d), 0, 0, 0);
        d += dd;
        u += du;
        if (d >= (uint32_t)ND) { d -= ND; ++u; }
    }
}

// Wait until this wave's LDS reads have returned (before the load unit may
// overwrite what they read).
__device__ __forceinline__ void wait_lds_reads() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Wait until at most N vector-memory operations of this wave are in flight
// (they complete in issue order).  N <= 15.
template <int N>
__device__ __forceinline__ void wait_vmem_at_most() { __builtin_amdgcn_s_waitcnt(0x0F70 | N); }

// Buffer loads issued by load_dwords<ND>.
template <int ND> constexpr int kDwordLoads = (ND - 1) / 4 + ((ND - 1) % 4 != 0) + 1;

// Corner data and weights of one sampling point, in flight.
template <int NV>
struct PointRegs {
    u32x4 v00[NV], v01[NV], v10[NV], v11[NV];
    float w00, w01, w10, w11;
};

// DCNv3-style weights of one unit (SM): w_k = exp(m_k - max) / sum_j exp(m_j -
// max), max and sum over the unit's P raw weights in point order; get(k)
// recomputes exp(m_k - max) (the same value as in the sum) and divides.  The
// same binary32 operations as the direct kernel's, so both families give
// the same weights; only the row and two floats stay in registers.
template <int P, typename Row>
struct SoftRow {
    Row r;
    float mx, rs;
    __device__ __forceinline__ explicit SoftRow(const Row& row) : r(row)
    {
        mx = r.get(0);
#pragma unroll
        for (int k = 1; k < P; ++k) mx = fmaxf(mx, r.get(k));
        rs = 0.0f;
#pragma unroll
        for (int k = 0; k < P; ++k) rs += expf(r.get(k) - mx);
    }
    __device__ __forceinline__ float get(int k) const { return expf(r.get(k) - mx) / rs; }
};

// Keep the compiler from moving memory operations across this point: bounds
// the number of sampling points whose corner reads are in flight per lane.
__device__ __forceinline__ void fence_sched() { asm volatile("" ::: "memory"); }

// Value barrier: the data of a point is taken as produced here, so the
// optimiser cannot hoist its widening (bf16) above the point's fence and keep
// both the raw and the widened copies alive.
template <int NV>
__device__ __forceinline__ void pin(PointRegs<NV>& r)
{
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        asm volatile("" : "+v"(r.v00[v]));
        asm volatile("" : "+v"(r.v01[v]));
        asm volatile("" : "+v"(r.v10[v]));
        asm volatile("" : "+v"(r.v11[v]));
    }
}

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>).
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

// Index of the n-th (from 0) set bit of m; n < popcount(m).
__device__ __forceinline__ uint32_t nth_set_bit(uint64_t m, int n)
{
    uint32_t pos = 0;
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) {
        const int c = __popcll(m & ((1ull << w) - 1));
        if (n >= c) {
            n -= c;
            m >>= w;
            pos += w;
        }
    }
    return pos;
}

// Per-workgroup constants the point steps need.
struct WinCtx {
    const char* lbase;
    __amdgpu_buffer_rsrc_t rx;
    float scale, fW, fH;
    int dil;
    float wx_lo, wx_hi, wy_lo, wy_hi;   // window test: wx_lo <= px < wx_hi, wy_lo <= py < wy_hi
    float zx, zy;                       // position of the zero columns (top-left corner)
    int zxi, zyi;                       // the same as integers
    int row16;                          // bytes per LDS row
    int xstep;                          // bytes between horizontally adjacent pixels
    int plane;                          // bytes per LDS plane
    int cbase;                          // LDS byte of image pixel (0,0) in plane 0
    uint32_t row_bytes, pix_bytes;      // global x strides
    int H, W;
};

// Point k (grid index q): weights, then the reads of its four corners from
// the LDS window.  A point that contributes nothing reads the window's zero
// columns with weight 0.  A valid point whose corners leave a partial window
// reads the zero columns too and sets `fb`: its whole unit is then
// recomputed from global memory by unit_global (same operation order).
template <int DT, int NV, int FULL, int RC, int P, int SPLIT, typename MR>
__device__ __forceinline__ PointRegs<NV> issue_point(const WinCtx& x, const RowLoad<DT, 2 * P>& offs,
                                                     const MR& msk, int k, int bx, int by,
                                                     int ubase, bool& fb)
{
    PointRegs<NV> r;
    const int q = (RC && k >= 4) ? k + 1 : k;
    const int i = q / 3, j = q % 3;
    float px = fmaf(offs.get(k), x.scale, (float)(bx + j * x.dil));
    float py = fmaf(offs.get(P + k), x.scale, (float)(by + i * x.dil));
    float m = msk.get(k);
    // bitwise & (not &&): no short-circuit, so no branch per point
    const bool valid = (px > -1.0f) & (px < x.fW) & (py > -1.0f) & (py < x.fH);
    bool ok = valid;
    if (!FULL) {
        const bool inwin = (px >= x.wx_lo) & (px < x.wx_hi) & (py >= x.wy_lo) & (py < x.wy_hi);
        ok = valid & inwin;
        fb = fb | (valid & !inwin);
    }
    // a point that reads nothing from the window sits on the zero columns
    // with weight 0: selecting positions, not addresses, keeps this branch-free
    px = ok ? px : x.zx;
    py = ok ? py : x.zy;
    m = ok ? m : 0.0f;
    const float fx = floorf(px), fy = floorf(py);
    const int x0 = (int)fx, y0 = (int)fy;
    const float lx = px - fx, ly = py - fy;
    const float hx = 1.0f - lx, hy = 1.0f - ly;
    const float mhy = m * hy, mly = m * ly;
    r.w00 = mhy * hx;
    r.w01 = mhy * lx;
    r.w10 = mly * hx;
    r.w11 = mly * lx;
    // ubase: the LDS byte of image pixel (0, 0) for the unit's vector 0 (it
    // may lie before the window, so it is added to the point's offset as an
    // integer: the corner's byte a00 is never negative, and every pointer
    // formed here stays inside the LDS allocation)
    const int a00 = __mul24(y0, x.row16) + (SPLIT ? __mul24(x0, x.xstep) : (x0 << 4)) + ubase;
    const char* p00 = x.lbase + a00;
    const char* p10 = p00 + x.row16;
    const int step01 = SPLIT ? x.xstep : 16;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const char* p0 = p00 + v * x.plane;
        const char* p1 = p10 + v * x.plane;
        r.v00[v] = *reinterpret_cast<const u32x4*>(p0);
        r.v01[v] = *reinterpret_cast<const u32x4*>(p0 + step01);
        r.v10[v] = *reinterpret_cast<const u32x4*>(p1);
        r.v11[v] = *reinterpret_cast<const u32x4*>(p1 + step01);
    }
    return r;
}

// Per channel, points in order, corners in the order 00, 01, 10, 11.  The
// accumulators are pinned afterwards: the multiply-adds of this point happen
// here, not sunk toward the store with the corner data kept alive.
template <int DT, int NV>
__device__ __forceinline__ void consume_point(float* acc, const PointRegs<NV>& r)
{
    constexpr int EPV = kPerVec<DT>;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        float* ac = acc + v * EPV;
        fma_vec16<DT>(ac, r.w00, r.v00[v]);
        fma_vec16<DT>(ac, r.w01, r.v01[v]);
        fma_vec16<DT>(ac, r.w10, r.v10[v]);
        fma_vec16<DT>(ac, r.w11, r.v11[v]);
    }
#pragma unroll
    for (int c = 0; c < NV * EPV; ++c) asm volatile("" : "+v"(acc[c]));
}

// Point k with its corners read from global memory (zero outside the image).
template <int DT, int NV, int RC, int P, typename MR>
__device__ __forceinline__ PointRegs<NV> issue_global(const WinCtx& x, const RowLoad<DT, 2 * P>& offs,
                                                      const MR& msk, int k, int bx, int by,
                                                      uint32_t gchan)
{
    const int q = (RC && k >= 4) ? k + 1 : k;
    const int i = q / 3, j = q % 3;
    const PointCoef c = point_coef(offs.get(k), offs.get(P + k), msk.get(k), x.scale,
                                   (float)(bx + j * x.dil), (float)(by + i * x.dil), x.fW, x.fH);
    const bool iny0 = c.valid & (c.y0 >= 0), iny1 = c.valid & (c.y0 + 1 < x.H);
    const bool inx0 = c.x0 >= 0, inx1 = c.x0 + 1 < x.W;
    const uint32_t b = (uint32_t)c.y0 * x.row_bytes + (uint32_t)c.x0 * x.pix_bytes + gchan;
    const uint32_t b01 = b + x.pix_bytes, b10 = b + x.row_bytes, b11 = b10 + x.pix_bytes;
    const uint32_t o00 = (iny0 & inx0) ? b : kOobOffset;
    const uint32_t o01 = (iny0 & inx1) ? b01 : kOobOffset;
    const uint32_t o10 = (iny1 & inx0) ? b10 : kOobOffset;
    const uint32_t o11 = (iny1 & inx1) ? b11 : kOobOffset;
    PointRegs<NV> r;
    r.w00 = c.w00; r.w01 = c.w01; r.w10 = c.w10; r.w11 = c.w11;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        r.v00[v] = buf_load16(x.rx, o00 + 16 * v);
        r.v01[v] = buf_load16(x.rx, o01 + 16 * v);
        r.v10[v] = buf_load16(x.rx, o10 + 16 * v);
        r.v11[v] = buf_load16(x.rx, o11 + 16 * v);
    }
    return r;
}

// The whole unit again, every corner read from global memory: the path for
// units with a point outside a partial window.  Same operation order as the
// fast path, so the result is the same sequence.
template <int DT, int NV, int RC, int P, typename MR>
__device__ __forceinline__ void unit_global(float* acc, const WinCtx& x, const RowLoad<DT, 2 * P>& offs,
                                            const MR& msk, int bx, int by, uint32_t gchan)
{
    constexpr int NC = NV * kPerVec<DT>;
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = 0.0f;
    // two points in flight, as in the main loop (the global reads' latency
    // would otherwise be paid once per point)
    PointRegs<NV> cur = issue_global<DT, NV, RC, P>(x, offs, msk, 0, bx, by, gchan);
#pragma unroll
    for (int k = 0; k < P; ++k) {
        PointRegs<NV> nxt;
        if (k + 1 < P) nxt = issue_global<DT, NV, RC, P>(x, offs, msk, k + 1, bx, by, gchan);
        fence_sched();
        pin(cur);
        consume_point<DT, NV>(acc, cur);
        fence_sched();
        cur = nxt;
    }
}

// Units split over SH lanes (SH = 2 or 4, so that a unit's lanes sit in one
// quad of lanes): the unit's P points are dealt to its lanes, lane v taking
// points v, v + SH, ...; each lane computes position, weights and corner
// address of its points only, and every point's are then broadcast to the
// unit's lanes with a quad permutation (DPP), instead of every lane
// computing all P points.  The operations and their order are the same as
// in issue_point, so the results are the same bits.
struct SlotCoef {
    float w00, w01, w10, w11;
    int a00;            // LDS byte of corner 00 for vector 0 of the unit
};

// Element e of a row when e depends on the lane: one of the SH candidates
// base .. base + SH - 1 (clamped to the row), chosen by v.
// (Each candidate passes through an empty asm: otherwise the optimiser turns
// the chain of selects into one load with a lane-dependent index, which puts
// the row in scratch memory.)
template <int SH, int NE, typename Row>
__device__ __forceinline__ float row_pick(const Row& r, int base, int v)
{
    float x = r.get(base < NE ? base : NE - 1);
    asm volatile("" : "+v"(x));
#pragma unroll
    for (int t = 1; t < SH; ++t) {
        const int e = base + t < NE ? base + t : NE - 1;
        float y = r.get(e);
        asm volatile("" : "+v"(y));
        x = v == t ? y : x;
    }
    return x;
}

// This lane's points' offsets and weights only (lane v of a unit computes
// points v, v + SH, ...; a slot past the unit's points reads point P - 1),
// one element load each, so that no lane holds the unit's whole rows or
// selects from them.  Same prefetch protocol as RowLoad: issue one unit
// ahead, read after the wait.
template <int DT, int P, int SH>
struct SlotRows {
    static constexpr int NS = (P + SH - 1) / SH;
    static constexpr uint32_t kEl = Elem<DT>::kBytes;
    uint32_t ox[NS], oy[NS], m[NS];

    static __device__ __forceinline__ uint32_t load_el(__amdgpu_buffer_rsrc_t r, uint32_t off)
    {
        if constexpr (kEl == 4) return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
        else return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
    }
    // so / sm: byte offsets of the unit's offset and weight rows; v: this
    // lane's place in its unit
    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t ro, __amdgpu_buffer_rsrc_t rm, uint32_t so,
                                          uint32_t sm, int v)
    {
#pragma unroll
        for (int t = 0; t < NS; ++t) {
            const uint32_t k = (uint32_t)min(t * SH + v, P - 1);
            ox[t] = load_el(ro, so + k * kEl);
            oy[t] = load_el(ro, so + ((uint32_t)P + k) * kEl);
            m[t] = load_el(rm, sm + k * kEl);
        }
    }
};

// Slot s of this lane (point k = s * SH + v): the steps of issue_point up to
// the corner address, from the point's x and y offsets and weight; `live` is
// false for a k past the unit's points.
template <int FULL, int RC, int P, int SH, int S>
__device__ __forceinline__ SlotCoef slot_coef_of(const WinCtx& x, float ox, float oy, float m, int v, int bx,
                                                 int by, int ubase, bool& fb)
{
    constexpr int s = S;
    const int k = s * SH + v;
    const bool live = k < P;
    const int q = k + ((RC && k >= 4) ? 1 : 0);
    const int i = (q * 11) >> 5, j = q - 3 * i;          // q / 3 and q % 3 for q < 10
    float px = fmaf(ox, x.scale, (float)(bx + j * x.dil));
    float py = fmaf(oy, x.scale, (float)(by + i * x.dil));
    const bool valid = (px > -1.0f) & (px < x.fW) & (py > -1.0f) & (py < x.fH);
    bool ok = valid;
    if (!FULL) {
        const bool inwin = (px >= x.wx_lo) & (px < x.wx_hi) & (py >= x.wy_lo) & (py < x.wy_hi);
        ok = valid & inwin;
        fb = fb | (live & valid & !inwin);
    }
    px = ok ? px : x.zx;
    py = ok ? py : x.zy;
    m = ok ? m : 0.0f;
    const float fx = floorf(px), fy = floorf(py);
    const int x0 = (int)fx, y0 = (int)fy;
    const float lx = px - fx, ly = py - fy;
    const float hx = 1.0f - lx, hy = 1.0f - ly;
    const float mhy = m * hy, mly = m * ly;
    SlotCoef c;
    c.w00 = mhy * hx;
    c.w01 = mhy * lx;
    c.w10 = mly * hx;
    c.w11 = mly * lx;
    c.a00 = __mul24(y0, x.row16) + __mul24(x0, x.xstep) + ubase;
    return c;
}

// The slot's values picked from the unit's whole rows (the softmax variant,
// whose weights need all of a unit's raw weights in every lane).
template <int DT, int FULL, int RC, int P, int SH, int S, typename MR>
__device__ __forceinline__ SlotCoef slot_coef(const WinCtx& x, const RowLoad<DT, 2 * P>& offs,
                                              const MR& msk, int v, int bx, int by, int ubase,
                                              bool& fb)
{
    return slot_coef_of<FULL, RC, P, SH, S>(x, row_pick<SH, 2 * P>(offs, S * SH, v),
                                            row_pick<SH, 2 * P>(offs, P + S * SH, v),
                                            row_pick<SH, P>(msk, S * SH, v), v, bx, by, ubase, fb);
}

// The slot's values from this lane's own loads.
template <int DT, int FULL, int RC, int P, int SH, int S>
__device__ __forceinline__ SlotCoef slot_coef(const WinCtx& x, const SlotRows<DT, P, SH>& sr, int v, int bx,
                                              int by, int ubase, bool& fb)
{
    using E = Elem<DT>;
    return slot_coef_of<FULL, RC, P, SH, S>(x, E::raw_to_f(sr.ox[S]), E::raw_to_f(sr.oy[S]),
                                            E::raw_to_f(sr.m[S]), v, bx, by, ubase, fb);
}

// Lane v of every unit's lane group takes lane `src` of the same group.
template <int SH, int SRC>
__device__ __forceinline__ int unit_bcast(int val)
{
    constexpr int a = SH == 4 ? SRC : SRC, b = SH == 4 ? SRC : SRC, c = SH == 4 ? SRC : 2 + SRC,
                  d = SH == 4 ? SRC : 2 + SRC;
    return __builtin_amdgcn_mov_dpp(val, a | (b << 2) | (c << 4) | (d << 6), 0xF, 0xF, true);
}

// Point k's corners for this lane's vectors, its weights taken from the
// lane that computed them.
// Shared coefficients need one group per workgroup, so a window pixel holds
// the unit's SH vectors and horizontally adjacent pixels are 16*SH bytes
// apart (an immediate offset of the corner reads).  vb: this lane's vector
// at LDS byte 0.
template <int NV, int SH, int K>
__device__ __forceinline__ PointRegs<NV> issue_shared(const WinCtx& x, const SlotCoef* sc, const char* vb)
{
    static_assert(NV == 1, "shared coefficients: one vector per lane");
    constexpr int S = K / SH, SRC = K % SH;
    constexpr int XS = 16 * SH;
    PointRegs<NV> r;
    r.w00 = __int_as_float(unit_bcast<SH, SRC>(__float_as_int(sc[S].w00)));
    r.w01 = __int_as_float(unit_bcast<SH, SRC>(__float_as_int(sc[S].w01)));
    r.w10 = __int_as_float(unit_bcast<SH, SRC>(__float_as_int(sc[S].w10)));
    r.w11 = __int_as_float(unit_bcast<SH, SRC>(__float_as_int(sc[S].w11)));
    const char* p0 = vb + unit_bcast<SH, SRC>(sc[S].a00);
    const char* p1 = p0 + x.row16;
    r.v00[0] = *reinterpret_cast<const u32x4*>(p0);
    r.v01[0] = *reinterpret_cast<const u32x4*>(p0 + XS);
    r.v10[0] = *reinterpret_cast<const u32x4*>(p1);
    r.v11[0] = *reinterpret_cast<const u32x4*>(p1 + XS);
    return r;
}

// SPLIT (with NV = 1, no coalesced rows): a.lpu consecutive lanes share a
// unit, lane v of them taking 16-byte vector v of the unit's channels (for
// units of many vectors, whose whole-unit registers would cap a workgroup at
// 512 threads).  The window then holds each pixel's vectors side by side,
// (row, column, vector), so that a unit's lanes read neighbouring entries.
template <int DT, int NV, int FULL, int RC, int COAL, int SPLIT, int SHARE, int SM, int MAXB>
__global__ void __launch_bounds__(MAXB)
k_window(KArgs a, uint32_t total_blocks, uint32_t per_xcd)
{
    static_assert(SHARE == 0 || (SPLIT && (SHARE == 2 || SHARE == 4)), "shared coefficients: split units");
    static_assert(!SPLIT || (NV == 1 && !COAL), "split units: one vector per lane, per-lane rows");
    using E = Elem<DT>;
    constexpr int s = E::kBytes;
    constexpr int EPV = kPerVec<DT>;          // elements per 16-byte vector
    constexpr int NC = NV * EPV;              // channels per lane (= Cg unless SPLIT)
    constexpr int P = 9 - RC;                 // points (K = 3)
    constexpr int ND = 2 * P * s / 4;         // dwords of one unit's offset row
    extern __shared__ u32x4 lds[];
    const uint32_t B = blockDim.x;
    const uint32_t lane = threadIdx.x & 63u;
    // per-wave buffers of the coalesced offset rows, after the window
    uint32_t* wbuf = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(lds) + a.win_bytes) +
                     (COAL ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * 64u * ND : 0u);

    uint32_t lb;
    if (!logical_block(blockIdx.x, total_blocks, per_xcd, &lb)) return;
    // logical block = ((n * tiles_y + ty) * tiles_x + tx) * gtiles + gt
    const uint32_t t1 = fdiv(lb, a.div_gtiles);
    const uint32_t gt = lb - t1 * a.gtiles;
    const uint32_t t2 = fdiv(t1, a.div_tiles_x);
    const uint32_t tx = t1 - t2 * a.tiles_x;
    const uint32_t n = fdiv(t2, a.div_tiles_y);
    const uint32_t ty = t2 - n * a.tiles_y;

    const int g0 = (int)gt * a.GB;
    const int oy0 = (int)ty * a.TH, ox0 = (int)tx * a.TW;
    const int wy0 = max(-1, oy0 * a.stride - a.pad - a.RY);
    const int wx0 = max(-1, ox0 * a.stride - a.pad - a.RX);
    const int wh = min(a.WH, a.H + 1 - wy0);  // window rows inside [-1, H]
    const int ww = min(a.WW, a.W + 1 - wx0);

    const char* xs = static_cast<const char*>(a.x) + (int64_t)n * a.img_x_elems * s;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(xs, a.img_x_bytes);
    const uint32_t pix_bytes = (uint32_t)a.C * s;
    const uint32_t row_bytes = (uint32_t)a.W * pix_bytes;
    const uint32_t grp_bytes = (uint32_t)(g0 * a.Cg) * s;

    const char* os_img = static_cast<const char*>(a.off) + (int64_t)n * a.img_off_elems * s;
    const char* ms_img = static_cast<const char*>(a.msk) + (int64_t)n * a.img_mask_elems * s;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(os_img, a.img_off_bytes);
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(ms_img, a.img_mask_bytes);
    const uint32_t units = (uint32_t)(a.TH * a.TW * a.GB);
    // lanes' work items: units, or (unit, vector) pairs when SPLIT
    const uint32_t lpu = SPLIT ? (uint32_t)a.lpu : 1u;
    const uint32_t items = units * lpu;
    auto unit_of_item = [&](uint32_t it) { return SPLIT ? fdiv(it, a.div_lpu) : it; };

    // unit u of this workgroup -> (pixel, group); its offset/weight rows are
    // prefetched one unit ahead
    auto unit_of = [&](uint32_t u, int& oy, int& ox, int& gl) {
        const uint32_t pl = fdiv(u, a.div_GB);
        gl = (int)(u - pl * (uint32_t)a.GB);
        const uint32_t oyl = fdiv(pl, a.div_TW);
        oy = oy0 + (int)oyl;
        ox = ox0 + (int)(pl - oyl * (uint32_t)a.TW);
    };
    auto row_starts = [&](int oy, int ox, int gl, uint32_t& so, uint32_t& sm) {
        const int64_t pix = (int64_t)oy * a.Wo + ox;
        const int g = g0 + gl;
        so = (uint32_t)((pix * a.off_row + (int64_t)g * 2 * P) * s);
        sm = (uint32_t)((pix * a.mask_row + (int64_t)g * P) * s);
    };

    RowLoad<DT, 2 * P> offs;
    RowLoad<DT, P> msk;
    // shared coefficients over four lanes (raw weights): each lane loads its
    // own points' values (stage-1 fp32: 66.5 -> 62.7 us, 116 -> 94 registers).
    // Units of two lanes keep the row loads: bfloat16 element loads measured
    // slower there (the 256x256 shape with sharing requested: 121.5 -> 128.8 us)
    constexpr bool kSlotRows = SHARE == 4 && !SM;
    SlotRows<DT, P, (SHARE ? SHARE : 1)> srows;
    if constexpr (kSlotRows) {
        // the row loads are not used on this path: defined values for the
        // copies below, which the compiler then drops
        offs = RowLoad<DT, 2 * P>{};
        msk = RowLoad<DT, P>{};
    }
    const int vshare = SHARE ? (int)(lane & (SHARE - 1)) : 0;
    // coalesced rows: with one group per workgroup and full-width tiles, unit
    // u of the tile is pixel oy0*Wo + u, so a wave's rows are evenly spaced
    const uint32_t off_row_bytes = (uint32_t)(a.off_row * s);
    const uint32_t off_tile_base = (uint32_t)(((int64_t)oy0 * a.Wo * a.off_row + (int64_t)g0 * 2 * P) * s);
    // linear bookkeeping (coalesced variant): unit u is pixel pix = oy0*Wo + u
    // of group g0, so moving a lane from unit u to u + B is a few additions
    // (rows beyond the image read as zeros and are never stored)
    int lin_oy = 0, lin_ox = 0;
    uint32_t lin_sm = 0, lin_oo = 0, lin_dox = 0, lin_doy = 0;
    const uint32_t mask_row_bytes = (uint32_t)(a.mask_row * s);
    if (COAL) {
        const uint32_t oyl = fdiv(threadIdx.x, a.div_TW);
        lin_oy = oy0 + (int)oyl;
        lin_ox = (int)(threadIdx.x - oyl * (uint32_t)a.Wo);
        const uint32_t pix = (uint32_t)(oy0 * a.Wo) + threadIdx.x;
        lin_sm = pix * mask_row_bytes + (uint32_t)(g0 * P * s);
        lin_oo = (pix * (uint32_t)a.C + (uint32_t)(g0 * a.Cg)) * s;
        lin_doy = fdiv(B, a.div_TW);
        lin_dox = B - lin_doy * (uint32_t)a.Wo;
    }
    // the first unit's offset and weight rows: requested right after the
    // window's loads (below), so that they queue behind them and stay in
    // flight across the barrier
    auto first_rows = [&]() {
        if (COAL) {
            stage_offset_rows<ND>(os_img, a.img_off_bytes, wbuf, lane,
                                  off_tile_base + (threadIdx.x - lane) * off_row_bytes, off_row_bytes);
            if (threadIdx.x < units) msk.issue(rm, lin_sm);
        } else if (threadIdx.x < items) {
            int oy, ox, gl;
            unit_of(unit_of_item(threadIdx.x), oy, ox, gl);
            uint32_t so, sm;
            row_starts(min(oy, a.Ho - 1), min(ox, a.Wo - 1), gl, so, sm);
            if constexpr (kSlotRows) {
                srows.issue(ro, rm, so, sm, vshare);
            } else {
                offs.issue(ro, so);
                msk.issue(rm, sm);
            }
        }
    };

    // ---- stage the window.  Chunk c = (window pixel p = c / CPS, chunk
    // cc = c % CPS of its CPS 16-byte chunks), read in that order (pixel-
    // contiguous in x) and written to plane cc at (row, col) of p (SPLIT:
    // to entry c).  Columns from WW to the pitch stay zero, as does
    // everything outside the image.
    const uint32_t CPS = (uint32_t)a.GB * (SPLIT ? (uint32_t)a.nvt : (uint32_t)NV);
    const uint32_t pitch = (uint32_t)a.pitch;
    const uint32_t plane16 = (uint32_t)a.WH * pitch;          // entries per plane
    const uint32_t nchunks = plane16 * CPS;
    {
        // U loads per lane in flight before their LDS writes: a whole-image
        // window of one group (about 7 chunks per lane) is staged in one round
        constexpr int U = 8;
        bool rows_issued = false;
        for (uint32_t c0 = threadIdx.x; c0 < nchunks || !rows_issued; c0 += B * U) {
            u32x4 v[U];
            uint32_t dst[U];
            // the wave's first chunk of this round (lane 0's), the same in every lane
            const uint32_t wc0 = __builtin_amdgcn_readfirstlane(c0 - lane);
#pragma unroll
            for (int r = 0; r < U; ++r) {
                const uint32_t c = c0 + r * B;
                // no chunk of the wave left in this slot: its address arithmetic
                // and load are skipped (a small window leaves most slots empty);
                // the LDS write below tests each lane's own chunk
                if (wc0 + r * B >= nchunks) continue;
                const uint32_t p = fdiv(c, a.div_CPS);
                const uint32_t cc = c - p * CPS;
                const uint32_t wyl = fdiv(p, a.div_pitch);
                const uint32_t wxl = p - wyl * pitch;
                const int y = wy0 + (int)wyl, x = wx0 + (int)wxl;
                const bool in = (c < nchunks) & (wxl < (uint32_t)a.WW) & (y >= 0) & (y < a.H) & (x >= 0) & (x < a.W);
                const uint32_t voff = (uint32_t)y * row_bytes + (uint32_t)x * pix_bytes + grp_bytes + cc * 16u;
                const uint32_t o = in ? voff : kOobOffset;
                v[r] = buf_load16(rx, o);
                dst[r] = SPLIT ? c : cc * plane16 + p;
            }
            if (!rows_issued) {
                fence_sched();
                first_rows();
                fence_sched();
                rows_issued = true;
            }
#pragma unroll
            for (int r = 0; r < U; ++r) {
                const uint32_t c = c0 + r * B;
                if (c < nchunks) lds[dst[r]] = v[r];
            }
        }
    }
    // the window's LDS writes are complete and visible to the workgroup; the
    // first rows' loads may still be in flight (no full memory fence here)
    wait_lds_reads();
    fence_sched();
    __builtin_amdgcn_s_barrier();
    fence_sched();

    WinCtx cx;
    cx.lbase = reinterpret_cast<const char*>(lds);
    cx.rx = rx;
    cx.scale = a.offset_scale;
    cx.fW = (float)a.W;
    cx.fH = (float)a.H;
    cx.dil = a.dil;
    cx.wx_lo = (float)wx0;
    cx.wx_hi = (float)(wx0 + ww - 1);
    cx.wy_lo = (float)wy0;
    cx.wy_hi = (float)(wy0 + wh - 1);
    cx.zxi = wx0 + a.WW;              // first zero column
    cx.zyi = wy0;
    cx.zx = (float)cx.zxi;
    cx.zy = (float)cx.zyi;
    cx.xstep = SPLIT ? (int)CPS * 16 : 16;
    cx.row16 = (int)pitch * cx.xstep;
    cx.plane = SPLIT ? 16 : (int)plane16 * 16;
    cx.cbase = -(wy0 * (int)pitch + wx0) * cx.xstep;
    cx.row_bytes = row_bytes;
    cx.pix_bytes = pix_bytes;
    cx.H = a.H;
    cx.W = a.W;

    uint32_t u = threadIdx.x;
    // units whose points leave a partial window, one bit per pass: finished
    // after the main loop, with every corner read from global memory
    uint64_t fbmask = 0;
    // One unit per lane.  NEXT: the unit's lane has another pass, whose rows
    // are requested during this one.  Coalesced variant: the passes with a
    // successor run in a loop whose loads and stores are the same on every
    // path, and the wave's last pass follows it; with the first unit's rows
    // waited for here, the compiler's own waits at the top of a unit then
    // leave its predecessor's stores in flight.
    if (COAL) wait_vmem_at_most<0>();
    auto unit_pass = [&](auto next_tag, uint32_t pass) {
        constexpr bool NEXT = decltype(next_tag)::value;
        int oy, ox, gl;
        if (COAL) {
            oy = lin_oy; ox = lin_ox; gl = 0;
        } else {
            unit_of(unit_of_item(u), oy, ox, gl);
        }
        // SPLIT: this lane's vector of the unit
        const uint32_t vsub = SPLIT ? u - unit_of_item(u) * lpu : 0u;
        RowLoad<DT, 2 * P> co = offs;
        if (!COAL && !kSlotRows) co.finish();
        SlotRows<DT, P, (SHARE ? SHARE : 1)> csr;
        if constexpr (kSlotRows) csr = srows;
        if (COAL) {
            // this pass's rows, staged by the wave one pass ahead.  Issued
            // since then, in this order (the fences keep it): the staging
            // loads, the weight-row loads (kMaskOps) and the previous unit's
            // stores (NV); waiting down to the smaller of the last two counts
            // leaves only later operations in flight
            constexpr int kMaskOps = kDwordLoads<RowLoad<DT, P>::kLoadDwords>;
            wait_vmem_at_most<(kMaskOps < NV ? kMaskOps : NV)>();
            fence_sched();
#pragma unroll
            for (int d = 0; d < ND; ++d) co.w[d] = wbuf[lane * ND + d];
            wait_lds_reads();
        }
        RowLoad<DT, P> cm = msk;
        if (!kSlotRows) cm.finish();
        // the rows just read are unpacked here, before the next unit's rows
        // are requested into the same registers: a read of them sunk below
        // that request would keep both sets alive and force a copy of rows in
        // flight at the end of the unit (a wait for every load and store)
        if (COAL) {
#pragma unroll
            for (int i = 0; i < RowLoad<DT, P>::kWords; ++i) asm volatile("" : "+v"(cm.w[i]));
        }

        // the next unit's rows are requested now and land while this unit
        // computes (without a per-lane test in the coalesced variant: rows
        // past the image read as zeros and are never used)
        uint32_t nso = 0, nsm = 0;
        const bool more = u + B < items;
        if (COAL && NEXT)
            stage_offset_rows<ND>(os_img, a.img_off_bytes, wbuf, lane, off_tile_base + (u - lane + B) * off_row_bytes,
                                  off_row_bytes);
        fence_sched();
        uint32_t oo = 0;
        if (COAL) {
            oo = lin_oo;
            if (NEXT) msk.issue(rm, lin_sm + B * mask_row_bytes);
            lin_sm += B * mask_row_bytes;
            lin_oo += B * (uint32_t)a.C * s;
            lin_ox += (int)lin_dox;
            lin_oy += (int)lin_doy;
            if (lin_ox >= a.Wo) { lin_ox -= a.Wo; ++lin_oy; }
        } else if (NEXT && more) {
            int oy2, ox2, gl2;
            unit_of(unit_of_item(u + B), oy2, ox2, gl2);
            row_starts(min(oy2, a.Ho - 1), min(ox2, a.Wo - 1), gl2, nso, nsm);
            if constexpr (kSlotRows) {
                srows.issue(ro, rm, nso, nsm, vshare);
            } else {
                offs.issue(ro, nso);
                msk.issue(rm, nsm);
            }
        }
        // (a whole-image window's units all lie inside the image)
        if (!FULL && (oy >= a.Ho || ox >= a.Wo)) return;
        const int g = g0 + gl;

        float acc[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[c] = 0.0f;

        const int bx = __mul24(ox, a.stride) - a.pad;
        const int by = __mul24(oy, a.stride) - a.pad;
        const int ubase = SPLIT ? (int)((gl * a.nvt + vsub) * 16u) + cx.cbase : gl * NV * cx.plane + cx.cbase;

        // the points' weights: the raw row, or its softmax (SM)
        const auto mrow = [&]() {
            if constexpr (SM) return SoftRow<P, RowLoad<DT, P>>(cm);
            else return cm;
        }();

        bool fb = false;
        if constexpr (SHARE) {
            // this lane's points, then every point broadcast within the unit;
            // two points in flight as below
            constexpr int NS = (P + SHARE - 1) / SHARE;
            const int v = (int)(lane & (SHARE - 1));
            const int ucommon = ubase - (int)(vsub * 16u);   // the unit's vector 0
            SlotCoef sc[NS];
            static_for<NS>([&](auto sic) {
                constexpr int si = decltype(sic)::value;
                if constexpr (kSlotRows)
                    sc[si] = slot_coef<DT, FULL, RC, P, SHARE, si>(cx, csr, v, bx, by, ucommon, fb);
                else
                    sc[si] = slot_coef<DT, FULL, RC, P, SHARE, si>(cx, co, mrow, v, bx, by, ucommon, fb);
            });
            if (!FULL) {
                // a unit is recomputed when any of its lanes found a point
                // outside the window
                int f = fb ? 1 : 0;
                f |= __builtin_amdgcn_mov_dpp(f, 0xB1, 0xF, 0xF, true);            // quad_perm [1,0,3,2]
                if (SHARE == 4) f |= __builtin_amdgcn_mov_dpp(f, 0x4E, 0xF, 0xF, true);   // [2,3,0,1]
                fb = f != 0;
            }
            const char* vb = cx.lbase + vsub * 16u;
            PointRegs<NV> cur = issue_shared<NV, SHARE, 0>(cx, sc, vb);
            static_for<P>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                PointRegs<NV> nxt;
                if constexpr (k + 1 < P) nxt = issue_shared<NV, SHARE, k + 1>(cx, sc, vb);
                fence_sched();
                pin(cur);
                consume_point<DT, NV>(acc, cur);
                fence_sched();
                cur = nxt;
            });
        } else {
            // two points in flight: issue the reads of point k+1, then accumulate point k
            PointRegs<NV> cur = issue_point<DT, NV, FULL, RC, P, SPLIT>(cx, co, mrow, 0, bx, by, ubase, fb);
#pragma unroll
            for (int k = 0; k < P; ++k) {
                PointRegs<NV> nxt;
                if (k + 1 < P) nxt = issue_point<DT, NV, FULL, RC, P, SPLIT>(cx, co, mrow, k + 1, bx, by, ubase, fb);
                fence_sched();
                pin(cur);
                consume_point<DT, NV>(acc, cur);
                fence_sched();
                cur = nxt;
            }
        }
        if (!FULL) fbmask |= (uint64_t)fb << pass;

        if (FULL) {
            char* op;
            if (COAL) {
                op = static_cast<char*>(a.out) + (int64_t)n * a.img_out_elems * s + oo;
            } else {
                const int64_t pix = (int64_t)oy * a.Wo + ox;
                op = static_cast<char*>(a.out) + ((int64_t)n * a.img_out_elems + pix * a.C + (int64_t)g * a.Cg) * s +
                     vsub * 16u;
            }
#pragma unroll
            for (int v = 0; v < NV; ++v)
                *reinterpret_cast<u32x4*>(op + 16 * v) = pack_vec16<DT>(acc + v * EPV);
        } else {
            // a unit marked in fbmask is recomputed and stored below, so its
            // store here goes to an offset out of the buffer's range, which the
            // hardware drops.  No branch: a store that depended on fb would let
            // the compiler sink every multiply-add of the unit below the branch
            // and keep all nine points' corner data alive at once
            const __amdgpu_buffer_rsrc_t rout =
                make_rsrc(static_cast<char*>(a.out) + (int64_t)n * a.img_out_elems * s, (uint32_t)(a.img_out_elems * s));
            const uint32_t at = COAL ? oo
                                     : (uint32_t)((((int64_t)oy * a.Wo + ox) * a.C + (int64_t)g * a.Cg) * s) + vsub * 16u;
            const uint32_t o = fb ? kOobOffset : at;
#pragma unroll
            for (int v = 0; v < NV; ++v)
                __builtin_amdgcn_raw_buffer_store_b128(pack_vec16<DT>(acc + v * EPV), rout, (int)(o + 16u * v), 0, 0);
        }
    };
    uint32_t pass = 0;
    if (COAL) {
        // u - lane: the wave's first unit of this pass (the same in every lane)
        for (; u - lane + B < units; u += B, ++pass) unit_pass(std::true_type{}, pass);
        if (u < units) unit_pass(std::false_type{}, pass);
    } else {
        // (per-lane requests of the next unit's rows, see `more`)
        for (; u < items; u += B, ++pass) unit_pass(std::true_type{}, pass);
    }

    if (!FULL) {
        // the wave's fallback items (item threadIdx.x + pass * B for bit
        // `pass` of a lane's fbmask), packed densely over its 64 lanes: a
        // batch of 64 costs one round of global reads, where each lane's own
        // items would cost a round per pass holding any of them
        auto fallback_item = [&](uint32_t it) {
            int oy, ox, gl;
            unit_of(unit_of_item(it), oy, ox, gl);
            const uint32_t vb = SPLIT ? (it - unit_of_item(it) * lpu) * 16u : 0u;   // this lane's vector
            const int g = g0 + gl;
            uint32_t so, sm;
            row_starts(oy, ox, gl, so, sm);
            RowLoad<DT, 2 * P> fo;
            RowLoad<DT, P> fm;
            fo.load(ro, so);
            fm.load(rm, sm);
            const auto fw = [&]() {
                if constexpr (SM) return SoftRow<P, RowLoad<DT, P>>(fm);
                else return fm;
            }();
            float acc[NC];
            unit_global<DT, NV, RC, P>(acc, cx, fo, fw, ox * a.stride - a.pad, oy * a.stride - a.pad,
                                       (uint32_t)(g * a.Cg) * s + vb);
            const int64_t pix = (int64_t)oy * a.Wo + ox;
            char* op = static_cast<char*>(a.out) + ((int64_t)n * a.img_out_elems + pix * a.C + (int64_t)g * a.Cg) * s + vb;
#pragma unroll
            for (int v = 0; v < NV; ++v)
                *reinterpret_cast<u32x4*>(op + 16 * v) = pack_vec16<DT>(acc + v * EPV);
        };
        const uint32_t npass = (items + B - 1) / B;
        const uint32_t wbase = threadIdx.x - lane;   // the wave's first thread
        uint32_t p = 0;                              // pass of the items in mp
        uint64_t mp = __ballot((int)(fbmask & 1u));  // its items not yet given out
        for (;;) {
            // a batch: lanes 0 .. fill - 1 take the next items, pass by pass
            int fill = 0;
            int my = -1;
            while (fill < 64) {
                while (!mp && ++p < npass) mp = __ballot((int)((fbmask >> p) & 1u));
                if (!mp) break;
                const int cnt = __popcll(mp);
                const int take = min(cnt, 64 - fill);
                const int nth = (int)lane - fill;
                if (nth >= 0 && nth < take) my = (int)(wbase + nth_set_bit(mp, nth) + p * B);
                mp = take < cnt ? mp & (~0ull << nth_set_bit(mp, take)) : 0ull;
                fill += take;
            }
            if (!fill) break;
            if (my >= 0) fallback_item((uint32_t)my);
        }
    }
}

}  // namespace

namespace {

template <int NV> constexpr int kMaxBlock = NV <= 2 ? 1024 : 512;

template <int SM, int DT, int NV, int FULL, int RC, int COAL, int SPLIT = 0, int SHARE = 0>
hipError_t launch5(const KArgs& a, int block, int64_t grid, hipStream_t stream)
{
    if (block > kMaxBlock<NV> || block < 64 || block % 64) return hipErrorInvalidValue;
    const uint32_t total = (uint32_t)grid;
    const uint32_t per_xcd = (total + 7) / 8;
    hipLaunchKernelGGL((k_window<DT, NV, FULL, RC, COAL, SPLIT, SHARE, SM, kMaxBlock<NV>>), dim3(per_xcd * 8),
                       dim3(block), a.lds_bytes, stream, a, total, per_xcd);
    return hipGetLastError();
}

template <int SM, int DT, int NV, int FULL, int RC>
hipError_t launch4(const KArgs& a, int block, int64_t grid, hipStream_t stream)
{
    return a.coal ? launch5<SM, DT, NV, FULL, RC, 1>(a, block, grid, stream)
                  : launch5<SM, DT, NV, FULL, RC, 0>(a, block, grid, stream);
}

// Units split over a.lpu lanes, one 16-byte vector each; units of 2 or 4
// lanes share their points' coefficients (SH), others compute them per lane.
template <int SM, int DT, int SH>
hipError_t launch_split_sh(const KArgs& a, int block, int64_t grid, hipStream_t stream)
{
    if (a.full)
        return a.remove_center ? launch5<SM, DT, 1, 1, 1, 0, 1, SH>(a, block, grid, stream)
                               : launch5<SM, DT, 1, 1, 0, 0, 1, SH>(a, block, grid, stream);
    return a.remove_center ? launch5<SM, DT, 1, 0, 1, 0, 1, SH>(a, block, grid, stream)
                           : launch5<SM, DT, 1, 0, 0, 0, 1, SH>(a, block, grid, stream);
}

template <int SM, int DT>
hipError_t launch_split(const KArgs& a, int block, int64_t grid, hipStream_t stream)
{
    if (a.coal || a.lpu < 2) return hipErrorInvalidValue;
    // shared coefficients address a window pixel's lpu vectors with a constant
    // step: one group per workgroup, as many vectors as lanes
    if (a.share && (a.GB != 1 || a.nvt != a.lpu)) return hipErrorInvalidValue;
    if (a.share && a.lpu == 4) return launch_split_sh<SM, DT, 4>(a, block, grid, stream);
    if (a.share && a.lpu == 2) return launch_split_sh<SM, DT, 2>(a, block, grid, stream);
    return launch_split_sh<SM, DT, 0>(a, block, grid, stream);
}

template <int SM, int DT, int NV>
hipError_t launch_nv(const KArgs& a, int block, int64_t grid, hipStream_t stream)
{
    if (a.full)
        return a.remove_center ? launch4<SM, DT, NV, 1, 1>(a, block, grid, stream)
                               : launch4<SM, DT, NV, 1, 0>(a, block, grid, stream);
    return a.remove_center ? launch4<SM, DT, NV, 0, 1>(a, block, grid, stream)
                           : launch4<SM, DT, NV, 0, 0>(a, block, grid, stream);
}

template <int SM, int DT>
hipError_t launch_dt(const KArgs& a, int nv, int block, int64_t grid, hipStream_t stream)
{
    if (a.lpu > 1) return launch_split<SM, DT>(a, block, grid, stream);
    switch (nv) {
        case 1: return launch_nv<SM, DT, 1>(a, block, grid, stream);
        case 2: return launch_nv<SM, DT, 2>(a, block, grid, stream);
        case 3: return launch_nv<SM, DT, 3>(a, block, grid, stream);
        case 4: return launch_nv<SM, DT, 4>(a, block, grid, stream);
        case 5: return launch_nv<SM, DT, 5>(a, block, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

// The window family's launch for one weight form (SM: softmax-normalised).
template <int SM>
hipError_t launch_window_form(const KArgs& a, int dtype, int nv, int block, int64_t grid, hipStream_t stream)
{
    switch (dtype) {
        case DCNV4_F32: return launch_dt<SM, DCNV4_F32>(a, nv, block, grid, stream);
        case DCNV4_F16: return launch_dt<SM, DCNV4_F16>(a, nv, block, grid, stream);
        case DCNV4_BF16: return launch_dt<SM, DCNV4_BF16>(a, nv, block, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

}  // namespace dcnv4

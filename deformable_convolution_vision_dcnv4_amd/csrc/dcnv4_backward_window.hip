// DCNv4 backward, offset and weight gradients with the corner reads served
// from an LDS copy of the image (the forward's window idea applied to the
// backward's gather).
//
// Gradients (the forward of jsqmd.com/news/933833, section 1, code example
// "DCNv4核心计算流程示例", with raw weights per the same section and
// bqwf.cn/news/1148139 section 2.1), per unit (pixel, group) and point k with
// bilinear fractions (lx, ly), hx = 1 - lx, hy = 1 - ly, and A_q = sum over
// the group's channels c of g_c * x[q]_c for the four corners q:
//   dL/dm_k         = hy hx A00 + hy lx A01 + ly hx A10 + ly lx A11
//   dL/doffset_x[k] = offset_scale * m_k * (hy (A01 - A00) + ly (A11 - A10))
//   dL/doffset_y[k] = offset_scale * m_k * (hx (A10 - A00) + lx (A11 - A01))
// (the per-channel expressions, summed over the channels first: four dot
// products per point instead of three sums of bilinear expressions per
// channel).  Points the forward skips get zero gradients.
//
// Work layout: one workgroup = (image n, output tile, group g).  A window of
// the zero-bordered image of that group is copied to LDS (one plane per
// 16-byte channel vector, rows of `pitch` entries): the whole image,
// [-1, H] x [-1, W], when it fits and the batch fills the GPU (one tile per
// image: every corner of every point is then in LDS), else the tile's grid
// with a margin, and a point whose corners leave the window reads them from
// global memory.  One lane = one (unit, point) with all of the group's
// channels.  Workgroups are renumbered per XCD so that a tile's groups, whose
// pixels share cache lines, meet in one L2.  The results are deterministic
// (a fixed operation order, whichever memory a corner comes from).

#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "dcnv4_device.h"
#include "dcnv4_internal.h"
#include "dcnv4_kernels.h"

namespace dcnv4 {
namespace {

// A += sum over the vector's elements e of g[e] * v_e, in element order.
template <int DT>
__device__ __forceinline__ float dot_vec16(float A, const float* g, u32x4 v)
{
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
    if constexpr (DT == DCNV4_F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) A = fmaf(g[i], __uint_as_float(d[i]), A);
    } else if constexpr (DT == DCNV4_F16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f16x2 h = __builtin_bit_cast(f16x2, d[i]);
            A = fmaf(g[2 * i], (float)h.x, A);
            A = fmaf(g[2 * i + 1], (float)h.y, A);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            A = fmaf(g[2 * i], bf16_lo(d[i]), A);
            A = fmaf(g[2 * i + 1], bf16_hi(d[i]), A);
        }
    }
    return A;
}

// One lane per (unit, point): the P lanes of a unit are consecutive, so the
// unit's P values of each gradient row are written by one store instruction
// as one contiguous piece (per-lane stores of a unit's whole row would touch
// a different cache line in every lane).  Each lane reads its point's offset
// pair and weight and the unit's output gradient (the same 16-byte vectors
// for the unit's P lanes).
template <int DT, int NV, int RC>
__global__ void __launch_bounds__(1024) k_backward_om_window(BArgs a, uint32_t total_blocks, uint32_t per_xcd)
{
    using E = Elem<DT>;
    constexpr int s = E::kBytes;
    constexpr int EPV = kPerVec<DT>;
    constexpr int P = 9 - RC;                  // points (K = 3)
    constexpr int UPW = 64 / P;                // units per wave (the last 64 % P lanes idle)
    extern __shared__ u32x4 lds[];
    const uint32_t B = blockDim.x;

    uint32_t lb;
    if (!logical_block(blockIdx.x, total_blocks, per_xcd, &lb)) return;
    // logical block = (n * tiles + t) * G + g: the groups of a tile, whose
    // pixels share cache lines, side by side
    const uint32_t nt = fdiv(lb, a.div_G);
    const uint32_t g = lb - nt * (uint32_t)a.G;
    const uint32_t ntiles = (uint32_t)(a.om_tiles_y * a.om_tiles_x);
    const uint32_t n = nt / ntiles, t = nt - n * ntiles;
    const int ty = (int)t / a.om_tiles_x, tx = (int)t - ty * a.om_tiles_x;
    const int oy0 = ty * a.om_th, ox0 = tx * a.om_tw;
    const int th = min(a.om_th, a.Ho - oy0), tw = min(a.om_tw, a.Wo - ox0);
    // the window: pixels [wy0, wy0 + wh) x [wx0, wx0 + ww) of the zero-bordered image
    const int wy0 = max(-1, oy0 * a.stride - a.pad - a.om_ry);
    const int wx0 = max(-1, ox0 * a.stride - a.pad - a.om_rx);
    const int wh = max(0, min(a.om_wh, a.H + 1 - wy0));
    const int ww = max(0, min(a.om_ww, a.W + 1 - wx0));

    const char* xs = static_cast<const char*>(a.x) + (int64_t)n * a.img_x_elems * s;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(xs, a.img_x_bytes);
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(static_cast<const char*>(a.off) + (int64_t)n * a.img_off_elems * s, a.img_off_bytes);
    const __amdgpu_buffer_rsrc_t rm =
        make_rsrc(static_cast<const char*>(a.msk) + (int64_t)n * a.img_mask_elems * s, a.img_mask_bytes);
    const __amdgpu_buffer_rsrc_t rg =
        make_rsrc(static_cast<const char*>(a.gout) + (int64_t)n * a.img_out_elems * s, a.img_out_bytes);
    const uint32_t pix_bytes = (uint32_t)a.C * s;
    const uint32_t row_bytes = (uint32_t)a.W * pix_bytes;
    const uint32_t grp_bytes = g * (uint32_t)a.Cg * s;

    // ---- staging: entry (plane v, row r, column c) holds pixel (wy0 + r,
    // wx0 + c), channels [v * EPV, v * EPV + EPV) of group g; zero off the
    // image.  Chunk q = pixel q / NV, plane q % NV: consecutive lanes read
    // consecutive 16-byte pieces of x.
    const uint32_t pitch = (uint32_t)a.pitch;
    const uint32_t plane16 = (uint32_t)a.om_wh * pitch;
    const uint32_t uww = (uint32_t)ww;
    const uint32_t nchunks = (uint32_t)wh * uww * NV;
    {
        constexpr int U = 8;
        for (uint32_t c0 = threadIdx.x; c0 < nchunks; c0 += B * U) {
            u32x4 v[U];
            uint32_t dst[U];
#pragma unroll
            for (int r = 0; r < U; ++r) {
                const uint32_t c = c0 + r * B;
                const uint32_t p = c / NV;
                const uint32_t cv = c - p * NV;
                const uint32_t wy = p / uww, wx = p - wy * uww;
                const int y = wy0 + (int)wy, x = wx0 + (int)wx;
                const bool in = (c < nchunks) & (y >= 0) & (y < a.H) & (x >= 0) & (x < a.W);
                const uint32_t voff = (uint32_t)y * row_bytes + (uint32_t)x * pix_bytes + grp_bytes + cv * 16u;
                v[r] = buf_load16(rx, in ? voff : kOobOffset);
                dst[r] = cv * plane16 + wy * pitch + wx;
            }
#pragma unroll
            for (int r = 0; r < U; ++r)
                if (c0 + r * B < nchunks) lds[dst[r]] = v[r];
        }
    }
    __syncthreads();

    const char* lbase = reinterpret_cast<const char*>(lds);
    const int row16 = (int)pitch * 16;
    const int plane = (int)plane16 * 16;
    const float fW = (float)a.W, fH = (float)a.H;
    // a point whose four corners lie in the window: wx0 <= px < wx0 + ww - 1 (same for y)
    const float wxl = (float)wx0, wxh = (float)(wx0 + ww - 1);
    const float wyl = (float)wy0, wyh = (float)(wy0 + wh - 1);
    const uint32_t units = (uint32_t)(th * tw);
    const float scale = a.offset_scale;

    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t ul = lane / P;              // unit within the wave
    const int k = (int)(lane - ul * P);        // point
    const int q = (RC && k >= 4) ? k + 1 : k;  // grid position of the point
    const int pi = q / 3, pj = q % 3;
    const uint32_t upass = (B >> 6) * UPW;     // units per pass of the workgroup
    for (uint32_t u0 = wave * UPW; u0 < units; u0 += upass) {
        const uint32_t ut = u0 + ul;
        if (ul >= UPW || ut >= units) continue;
        // row within the tile (the last tile of a row may be narrower)
        const uint32_t ry = tw == a.om_tw ? fdiv(ut, a.div_om_tw) : ut / (uint32_t)tw;
        const uint32_t oy = (uint32_t)oy0 + ry;
        const uint32_t ox = (uint32_t)ox0 + (ut - ry * (uint32_t)tw);
        const uint32_t u = oy * (uint32_t)a.Wo + ox;
        const int64_t prow = (int64_t)u * a.off_row + (int64_t)g * 2 * P;     // within the image
        const int64_t mrow = (int64_t)u * a.mask_row + (int64_t)g * P;
        float dx, dy, m;
        if constexpr (s == 4) {
            dx = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ro, (int)((prow + k) * 4), 0, 0));
            dy = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ro, (int)((prow + P + k) * 4), 0, 0));
            m = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rm, (int)((mrow + k) * 4), 0, 0));
        } else {
            dx = E::raw_to_f(__builtin_amdgcn_raw_buffer_load_b16(ro, (int)((prow + k) * 2), 0, 0));
            dy = E::raw_to_f(__builtin_amdgcn_raw_buffer_load_b16(ro, (int)((prow + P + k) * 2), 0, 0));
            m = E::raw_to_f(__builtin_amdgcn_raw_buffer_load_b16(rm, (int)((mrow + k) * 2), 0, 0));
        }
        u32x4 gv[NV];
        const uint32_t go = (u * (uint32_t)a.C + g * (uint32_t)a.Cg) * s;
#pragma unroll
        for (int v = 0; v < NV; ++v) gv[v] = buf_load16(rg, go + 16u * v);

        const float px = fmaf(dx, scale, (float)((int)ox * a.stride - a.pad + pj * a.dil));
        const float py = fmaf(dy, scale, (float)((int)oy * a.stride - a.pad + pi * a.dil));
        const bool valid = (px > -1.0f) & (px < fW) & (py > -1.0f) & (py < fH);
        const bool inwin = (px >= wxl) & (px < wxh) & (py >= wyl) & (py < wyh);
        const float pxs = valid ? px : wxl, pys = valid ? py : wyl;
        const float fx = floorf(pxs), fy = floorf(pys);
        const float lx = pxs - fx, ly = pys - fy;
        const float hx = 1.0f - lx, hy = 1.0f - ly;
        const int x0 = (int)fx, y0 = (int)fy;
        // window entry of corner (y0, x0); a point outside the window reads
        // entry 0 (a valid one then reads its corners from global memory,
        // a skipped one's gradients are zero whatever it reads)
        const int a00 = (valid & inwin) ? (y0 - wy0) * row16 + ((x0 - wx0) << 4) : 0;
        // corners from global memory (zero off the image) when the point is
        // valid but leaves the window
        const bool glob = valid & !inwin;
        const bool iny0 = y0 >= 0, iny1 = y0 + 1 < a.H, inx0 = x0 >= 0, inx1 = x0 + 1 < a.W;
        const uint32_t gbase = (uint32_t)y0 * row_bytes + (uint32_t)x0 * pix_bytes + grp_bytes;
        const uint32_t goffs[4] = {(iny0 & inx0) ? gbase : kOobOffset,
                                   (iny0 & inx1) ? gbase + pix_bytes : kOobOffset,
                                   (iny1 & inx0) ? gbase + row_bytes : kOobOffset,
                                   (iny1 & inx1) ? gbase + row_bytes + pix_bytes : kOobOffset};
        // vectors whose corners are held at once: all of them for units of
        // one or two vectors, one at a time for wider units (registers)
        constexpr int VC = NV <= 2 ? NV : 1;
        float A00 = 0.0f, A01 = 0.0f, A10 = 0.0f, A11 = 0.0f;
#pragma unroll
        for (int v0 = 0; v0 < NV; v0 += VC) {
            u32x4 cv[VC][4];
#pragma unroll
            for (int j = 0; j < VC; ++j) {
                const char* p0 = lbase + a00 + (v0 + j) * plane;
                cv[j][0] = *reinterpret_cast<const u32x4*>(p0);
                cv[j][1] = *reinterpret_cast<const u32x4*>(p0 + 16);
                cv[j][2] = *reinterpret_cast<const u32x4*>(p0 + row16);
                cv[j][3] = *reinterpret_cast<const u32x4*>(p0 + row16 + 16);
            }
            if (glob) {
#pragma unroll
                for (int j = 0; j < VC; ++j) {
#pragma unroll
                    for (int cr = 0; cr < 4; ++cr)
                        cv[j][cr] = buf_load16(rx, goffs[cr] == kOobOffset ? kOobOffset : goffs[cr] + 16u * (v0 + j));
                }
            }
#pragma unroll
            for (int j = 0; j < VC; ++j) {
                float gr[EPV];
                const u32x4 gvv = gv[v0 + j];
                const uint32_t w[4] = {gvv.x, gvv.y, gvv.z, gvv.w};
#pragma unroll
                for (int e = 0; e < EPV; ++e) {
                    if constexpr (s == 4) gr[e] = __uint_as_float(w[e]);
                    else gr[e] = E::raw_to_f((e & 1) ? (w[e / 2] >> 16) : (w[e / 2] & 0xffffu));
                }
                A00 = dot_vec16<DT>(A00, gr, cv[j][0]);
                A01 = dot_vec16<DT>(A01, gr, cv[j][1]);
                A10 = dot_vec16<DT>(A10, gr, cv[j][2]);
                A11 = dot_vec16<DT>(A11, gr, cv[j][3]);
            }
            // wide units: the next vector's reads are not hoisted above these
            // products (that would hold every vector's corners at once)
            if constexpr (VC < NV) asm volatile("" ::: "memory");
        }
        float sm = (hy * hx) * A00;
        sm = fmaf(hy * lx, A01, sm);
        sm = fmaf(ly * hx, A10, sm);
        sm = fmaf(ly * lx, A11, sm);
        const float sx = fmaf(hy, A01 - A00, ly * (A11 - A10));
        const float sy = fmaf(hx, A10 - A00, lx * (A11 - A01));
        const float ms = scale * m;
        if (a.goff) {
            float* gop = a.goff + (int64_t)n * a.img_off_elems + prow;
            gop[k] = valid ? ms * sx : 0.0f;
            gop[P + k] = valid ? ms * sy : 0.0f;
        }
        if (a.gmask) a.gmask[(int64_t)n * a.img_mask_elems + mrow + k] = valid ? sm : 0.0f;
    }
}

template <int DT, int NV>
void launch_rc(const BArgs& a, int block, uint32_t total, size_t lds, hipStream_t stream)
{
    const uint32_t per_xcd = (total + 7) / 8;
    if (a.remove_center)
        hipLaunchKernelGGL((k_backward_om_window<DT, NV, 1>), dim3(per_xcd * 8), dim3(block), lds, stream, a,
                           total, per_xcd);
    else
        hipLaunchKernelGGL((k_backward_om_window<DT, NV, 0>), dim3(per_xcd * 8), dim3(block), lds, stream, a,
                           total, per_xcd);
}

template <int DT>
hipError_t launch_nv(const BArgs& a, int nv, int block, uint32_t total, size_t lds, hipStream_t stream)
{
    switch (nv) {
        case 1: launch_rc<DT, 1>(a, block, total, lds, stream); break;
        case 2: launch_rc<DT, 2>(a, block, total, lds, stream); break;
        case 3: launch_rc<DT, 3>(a, block, total, lds, stream); break;
        case 4:
            if constexpr (DT != DCNV4_BF16) {
                launch_rc<DT, 4>(a, block, total, lds, stream);
                break;
            }
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

bool backward_om_window_plan(const Problem& p, const void* gout, OmPlan* plan)
{
    const int s = p.dtype == DCNV4_F32 ? 4 : 2;
    if (p.K != 3 || (p.Cg * s) % 16) return false;
    const int nv = p.Cg * s / 16;
    // units of up to four vectors (three in bf16, whose widening takes more
    // registers): wider ones spilled, and the latent shape's five bf16
    // vectors measured no faster than k_backward (138 us either way)
    if (nv > (p.dtype == DCNV4_BF16 ? 3 : 4)) return false;
    if ((uintptr_t)p.x % 16 || (uintptr_t)gout % 16) return false;
    // the whole zero-bordered image when it fits, rows a whole number of
    // 16-entry bank groups apart (as the forward's windows)
    OmPlan o;
    o.pitch = (p.W + 2 + 15) / 16 * 16;
    int64_t bytes = (int64_t)(p.H + 2) * o.pitch * nv * 16;
    // one workgroup per (image, group) holds a CU for the whole image: with
    // fewer of them than CUs (small batches), square tiles sized to fill the GPU
    const bool fill = backward_fill_gpu() && (int64_t)p.N * p.G < p.cus;
    if (bytes <= kLdsPerCu && !fill) {
        o.th = p.Ho;
        o.tw = p.Wo;
        o.ry = o.rx = p.pad + 1;              // the window starts at pixel -1
        o.wh = p.H + 2;
        o.ww = p.W + 2;
        const int64_t units = (int64_t)p.Ho * p.Wo;
        o.block = (int)(units < 1024 ? (units + 63) / 64 * 64 : 1024);
    } else {
        // tiles of th x tw units; the window covers their grid and r pixels
        // around it, points beyond read their corners from global memory.
        // DCNV4_BWD_OM="<th>,<tw>,<r>" overrides the shape (1..256, 0..64).
        // Units wider than the LDS allows at 32 x 32 take smaller square tiles.
        int th = 32, tw = 32, r = 8;
        bool shrink = true;
        if (fill) {
            const double t = sqrt((double)p.Ho * p.Wo * p.N * p.G / p.cus);
            th = tw = t < 4.0 ? 4 : t > 32.0 ? 32 : (int)t;
        }
        if (const char* env = getenv("DCNV4_BWD_OM")) {
            int eh = 0, ew = 0, er = -1;
            if (sscanf(env, "%d,%d,%d", &eh, &ew, &er) == 3 && eh >= 1 && eh <= 256 && ew >= 1 && ew <= 256 &&
                er >= 0 && er <= 64) {
                th = eh;
                tw = ew;
                r = er;
                shrink = false;
            }
        }
        for (;;) {
            o.th = th < p.Ho ? th : p.Ho;
            o.tw = tw < p.Wo ? tw : p.Wo;
            o.ry = o.rx = r;
            const int64_t eh = (int64_t)(o.th - 1) * p.stride + 2 * p.dil + 2 + 2 * r;
            const int64_t ew = (int64_t)(o.tw - 1) * p.stride + 2 * p.dil + 2 + 2 * r;
            o.wh = (int)(eh < p.H + 2 ? eh : p.H + 2);
            o.ww = (int)(ew < p.W + 2 ? ew : p.W + 2);
            o.pitch = (o.ww + 15) / 16 * 16;
            bytes = (int64_t)o.wh * o.pitch * nv * 16;
            if (bytes <= kLdsPerCu) break;
            if (!shrink || (th <= 4 && tw <= 4)) return false;
            th = th * 3 / 4 > 4 ? th * 3 / 4 : 4;
            tw = tw * 3 / 4 > 4 ? tw * 3 / 4 : 4;
        }
        // enough waves for one pass over the tile's (unit, point) lanes
        const int64_t waves = ((int64_t)o.th * o.tw + (64 / p.P) - 1) / (64 / p.P);
        o.block = (int)(waves < 16 ? waves * 64 : 1024);
    }
    o.tiles_y = (p.Ho + o.th - 1) / o.th;
    o.tiles_x = (p.Wo + o.tw - 1) / o.tw;
    o.lds = (size_t)bytes;
    *plan = o;
    return true;
}

hipError_t launch_backward_om_window(const BArgs& a, int dtype, int nv, int block, size_t lds,
                                     hipStream_t stream)
{
    // images x tiles x groups
    const uint32_t total = (uint32_t)(a.units_total / a.units_img) * (uint32_t)(a.om_tiles_y * a.om_tiles_x) *
                           (uint32_t)a.G;
    switch (dtype) {
        case DCNV4_F32: return launch_nv<DCNV4_F32>(a, nv, block, total, lds, stream);
        case DCNV4_F16: return launch_nv<DCNV4_F16>(a, nv, block, total, lds, stream);
        case DCNV4_BF16: return launch_nv<DCNV4_BF16>(a, nv, block, total, lds, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dcnv4

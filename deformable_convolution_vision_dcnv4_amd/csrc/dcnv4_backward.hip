// DCNv4 backward: gradients of the forward with respect to x, the offsets and
// the dynamic weights.
//
// The forward (jsqmd.com/news/933833, section 1, code example
// "DCNv4核心计算流程示例"; raw weights per the same section and
// bqwf.cn/news/1148139 section 2.1) is, per output channel,
//   out = sum_k m_k * sum_q tri(py_k - qy) tri(px_k - qx) x[q]
// over the bilinear corners q of point k, with tri(t) = max(0, 1 - |t|) and
// p_k = base_k + offset_scale * offset_k.  Its gradients, given g = dL/dout:
//   dL/dx[q]        += m_k * w_q(k) * g                      (scatter)
//   dL/dm_k          = sum_c g_c * sample_k,c
//   dL/doffset_x[k]  = offset_scale * m_k * sum_c g_c * (hy (x01 - x00) + ly (x11 - x10))
//   dL/doffset_y[k]  = offset_scale * m_k * sum_c g_c * (hx (x10 - x00) + lx (x11 - x01))
// (the derivative from the right at integer coordinates, which belongs to
// the corners floor(p), floor(p)+1 the forward uses).  Points the forward
// skips get zero gradient.
//
// Kernels here: k_backward, the general one (any K, any width), and for K = 3
// x's gradient in LDS, k_backward_x (a channel chunk of the whole bordered
// image) or k_backward_x_tiled (64 x 64 down to 8 x 8 tiles, for images too
// large for LDS or batches too small to fill the GPU); the offset and weight
// gradients of K = 3 come from the LDS-window kernel of
// dcnv4_backward_window.hip when it applies.
//
// k_backward's layout: as the forward's direct kernel, lanes take (unit,
// vector) pairs, unit = (pixel, group), L = Cg*s/VB lanes per unit, the L
// lanes of a unit in one wave.  Per point, each lane forms its channels'
// partial sums; the unit's first lane adds the L partials in lane order (a
// fixed order: the offset and weight gradients are reproducible) and writes
// them.  Its x's gradient (other K) is a scatter: hardware fp32 atomic adds
// into a buffer this library zeroes first (summation order not fixed).

#include <stdio.h>
#include <stdlib.h>
#include <string.h>


#include "dcnv4_device.h"
#include "dcnv4_internal.h"
#include "dcnv4_kernels.h"

namespace dcnv4 {
namespace {

__global__ void __launch_bounds__(256) k_zero_f32(float* __restrict__ p, int64_t n)
{
    const int64_t n4 = n / 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    float4* p4 = reinterpret_cast<float4*>(p);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
        p4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t i = n4 * 4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        p[i] = 0.f;
}

template <int VB>
__device__ __forceinline__ void load_vec(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t* d)
{
    if constexpr (VB == 16) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    } else if constexpr (VB == 8) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, 0, 0);
        d[0] = v.x; d[1] = v.y;
    } else if constexpr (VB == 4) {
        d[0] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, 0, 0);
    } else {
        d[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, 0, 0);
    }
}

// Element i (< VB / s) of a loaded vector, widened to binary32.
template <int DT>
__device__ __forceinline__ float elem(const uint32_t* d, int i)
{
    if constexpr (DT == DCNV4_F32) {
        return __uint_as_float(d[i]);
    } else {
        const uint32_t w = d[i / 2];
        return Elem<DT>::raw_to_f((i & 1) ? (w >> 16) : (w & 0xffffu));
    }
}

// Sum of v over the L lanes of this lane's unit, in lane order, valid in the
// unit's first lane (lane0 = that lane's index in the wave).
__device__ __forceinline__ float unit_sum(float v, int L, int lane0)
{
    float s = __shfl(v, lane0);
    for (int i = 1; i < L; ++i) s += __shfl(v, lane0 + i);
    return s;
}

template <int DT, int VB, int KT>
__global__ void __launch_bounds__(256) k_backward(BArgs a, uint32_t total_blocks, uint32_t per_xcd)
{
    using E = Elem<DT>;
    using S = typename E::S;
    constexpr int s = E::kBytes;
    constexpr int NE = VB / s;                 // channels per lane
    constexpr int NW = (VB + 3) / 4;           // dwords per vector

    // block = 4 waves; a wave holds upw units of L lanes (the rest idle)
    const int L = a.lanes;
    const int upw = a.units_per_wave;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int uiw = lane / L;                  // unit in wave
    const int lane_in_unit = lane - uiw * L;
    // blocks renumbered per XCD as in the direct forward kernel (per_xcd > 0)
    uint32_t lb = blockIdx.x;
    if (per_xcd && !logical_block(blockIdx.x, total_blocks, per_xcd, &lb)) return;
    const int64_t ublk = (int64_t)lb * 4 * upw;
    const int64_t unit_g = ublk + (int64_t)wave * upw + uiw;
    const bool active = uiw < upw && unit_g < a.units_total;
    const int lane0 = uiw * L;

    // unit -> (n, ho, wo, g); inactive lanes take unit 0 (all loads in range)
    const uint32_t u = active ? (uint32_t)unit_g : 0u;
    const uint32_t n = fdiv(u, a.div_units_img);
    const uint32_t ui = u - n * a.units_img;
    const uint32_t pix = fdiv(ui, a.div_G);
    const uint32_t g = ui - pix * (uint32_t)a.G;
    const uint32_t ho = fdiv(pix, a.div_Wo);
    const uint32_t wo = pix - ho * (uint32_t)a.Wo;

    const char* xs = static_cast<const char*>(a.x) + (int64_t)n * a.img_x_elems * s;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(xs, a.img_x_bytes);
    const S* os = static_cast<const S*>(a.off) + (int64_t)n * a.img_off_elems + (int64_t)pix * a.off_row + g * 2 * a.P;
    const S* ms = static_cast<const S*>(a.msk) + (int64_t)n * a.img_mask_elems + (int64_t)pix * a.mask_row + g * a.P;
    const uint32_t chan = g * (uint32_t)a.Cg + (uint32_t)(lane_in_unit * NE);
    const uint32_t pix_bytes = (uint32_t)a.C * s;
    const uint32_t row_bytes = (uint32_t)a.W * pix_bytes;

    // this lane's channels of the output gradient
    float gr[NE];
    {
        const S* gp = static_cast<const S*>(a.gout) + (int64_t)n * a.img_out_elems + (int64_t)pix * a.C + chan;
#pragma unroll
        for (int c = 0; c < NE; ++c) gr[c] = E::to_f(gp[c]);
    }
    float* gxi = a.gx ? a.gx + (int64_t)n * a.img_x_elems : nullptr;

    const float fW = (float)a.W, fH = (float)a.H;
    const int bx0 = (int)wo * a.stride - a.pad;
    const int by0 = (int)ho * a.stride - a.pad;
    const int K = KT > 0 ? KT : a.K, KK = K * K, center = KK / 2;
    constexpr int kUnroll = KT > 0 ? KT * KT : 1;
#pragma unroll kUnroll
    for (int q = 0; q < (KT > 0 ? KT * KT : KK); ++q) {
        if (a.remove_center && q == center) continue;
        const int k = (a.remove_center && q > center) ? q - 1 : q;
        const int i = q / K, j = q - (q / K) * K;
        const float dx = E::to_f(os[k]), dy = E::to_f(os[a.P + k]), m = E::to_f(ms[k]);
        float px = fmaf(dx, a.offset_scale, (float)(bx0 + j * a.dil));
        float py = fmaf(dy, a.offset_scale, (float)(by0 + i * a.dil));
        const bool valid = (px > -1.0f) & (px < fW) & (py > -1.0f) & (py < fH);
        px = valid ? px : 0.0f;
        py = valid ? py : 0.0f;
        const float fx = floorf(px), fy = floorf(py);
        const int x0 = (int)fx, y0 = (int)fy;
        const float lx = px - fx, ly = py - fy;
        const float hx = 1.0f - lx, hy = 1.0f - ly;

        const bool iny0 = valid & (y0 >= 0), iny1 = valid & (y0 + 1 < a.H);
        const bool inx0 = x0 >= 0, inx1 = x0 + 1 < a.W;
        const uint32_t base = (uint32_t)y0 * row_bytes + (uint32_t)x0 * pix_bytes + chan * s;
        const uint32_t b01 = base + pix_bytes, b10 = base + row_bytes, b11 = b10 + pix_bytes;
        uint32_t d00[NW], d01[NW], d10[NW], d11[NW];
        load_vec<VB>(rx, (iny0 & inx0) ? base : kOobOffset, d00);
        load_vec<VB>(rx, (iny0 & inx1) ? b01 : kOobOffset, d01);
        load_vec<VB>(rx, (iny1 & inx0) ? b10 : kOobOffset, d10);
        load_vec<VB>(rx, (iny1 & inx1) ? b11 : kOobOffset, d11);

        float sm = 0.0f, sx = 0.0f, sy = 0.0f;
#pragma unroll
        for (int c = 0; c < NE; ++c) {
            const float v00 = elem<DT>(d00, c), v01 = elem<DT>(d01, c);
            const float v10 = elem<DT>(d10, c), v11 = elem<DT>(d11, c);
            const float bil = hy * (hx * v00 + lx * v01) + ly * (hx * v10 + lx * v11);
            const float ddx = hy * (v01 - v00) + ly * (v11 - v10);
            const float ddy = hx * (v10 - v00) + lx * (v11 - v01);
            sm += gr[c] * bil;
            sx += gr[c] * ddx;
            sy += gr[c] * ddy;
        }

        // x's gradient: the forward's weights (m folded in) times g, per corner inside
        if (gxi && active && valid) {
            const float mhy = m * hy, mly = m * ly;
            const float w[4] = {mhy * hx, mhy * lx, mly * hx, mly * lx};
            const bool in[4] = {(bool)(iny0 & inx0), (bool)(iny0 & inx1), (bool)(iny1 & inx0), (bool)(iny1 & inx1)};
            const uint32_t off[4] = {base, b01, b10, b11};
#pragma unroll
            for (int cr = 0; cr < 4; ++cr) {
                if (!in[cr]) continue;
                float* dst = gxi + off[cr] / s;
#pragma unroll
                for (int c = 0; c < NE; ++c) unsafeAtomicAdd(dst + c, w[cr] * gr[c]);
            }
        }

        // the unit's sums, in lane order, by its first lane
        const float tm = unit_sum(sm, L, lane0);
        const float tx = unit_sum(sx, L, lane0);
        const float ty = unit_sum(sy, L, lane0);
        if (active && lane_in_unit == 0) {
            const float ms_ = valid ? a.offset_scale * m : 0.0f;
            const int64_t prow = (int64_t)n * a.img_off_elems + (int64_t)pix * a.off_row + g * 2 * a.P;
            const int64_t mrow = (int64_t)n * a.img_mask_elems + (int64_t)pix * a.mask_row + g * a.P;
            if (a.goff) {
                a.goff[prow + k] = valid ? ms_ * tx : 0.0f;
                a.goff[prow + a.P + k] = valid ? ms_ * ty : 0.0f;
            }
            if (a.gmask) a.gmask[mrow + k] = valid ? tm : 0.0f;
        }
    }
}

// x's gradient of one (image, group, chunk of CC channels), accumulated in an
// LDS copy of the zero-bordered image [-1, H] x [-1, W] (one plane per
// channel): every corner of every valid point lands inside it, corners off
// the image land on the border, which is dropped.  The workgroup owns that
// slice of grad_x, so it is written once with plain stores: no global
// atomics and no separate zeroing.
//
// The accumulation is in 64-bit fixed point with LDS integer atomic adds
// (binary32 LDS atomic adds run tens of times slower on this GPU).  Each
// term w * g (the exact product of the binary32 factors) becomes
// rint(w * g * 2^F); F is fixed per (image, group) so that no sum can overflow:
// with M = max|m| * max|g| over the (image, group) (|t| <= M) and at most
// 2^cbits terms per element, F = 62 - cbits - e where M < 2^e (at most
// 51 - e, which keeps every term below 2^51).  Integer sums
// do not depend on the order of the adds, so x's gradient is reproducible;
// each term is off by at most 2^-(F+1).  An (image, group) whose weights or
// output gradient hold a non-finite value uses binary32 LDS atomic adds.
// Static LDS of the x-gradient kernels: per-wave maxima and non-finite flags
// of a 1024-thread workgroup.  The planners reserve kBwdXStaticLds for it.
struct BxShared {
    float red[2][16];
    bool flag[16];
};
static_assert(sizeof(BxShared) <= kBwdXStaticLds, "static LDS of the x-gradient kernels");

// The units of a whole-image x-gradient workgroup in a spread order: index it takes
// unit (it % 32) * (n / 32) + it / 32 (a bijection of the first 32 * (n / 32)
// indices; the rest in order), so that consecutive lanes take units n / 32
// apart.  With small offsets, neighbouring units' corners would often hit the
// same or neighbouring accumulators in one atomic instruction (serialised
// adds and bank conflicts): stage-1 f16 backward 327 -> 291 us (spreads of 8
// and 128: 299 and 296 us; the tiled kernel measured no different with it).
// The fixed-point sums do not depend on the order.
__device__ __forceinline__ int spread_index(int it, int n)
{
    constexpr int kSpread = 32;
    const int q = n / kSpread;
    return it < kSpread * q ? (it % kSpread) * q + it / kSpread : it;
}

template <int DT, int RC, int CC>
__global__ void __launch_bounds__(1024) k_backward_x(BArgs a, uint32_t total_blocks, uint32_t per_xcd)
{
    using E = Elem<DT>;
    constexpr int s = E::kBytes;
    constexpr int P = 9 - RC;                 // K = 3
    extern __shared__ unsigned long long acc[];
    __shared__ BxShared sh_;
    float (&red)[2][16] = sh_.red;
    bool (&flag)[16] = sh_.flag;
    const int chunks = a.Cg / CC;
    // renumbered so that each XCD runs a contiguous range: the groups of an
    // image, whose rows share cache lines, meet in one L2
    uint32_t b;
    if (!logical_block(blockIdx.x, total_blocks, per_xcd, &b)) return;
    const uint32_t n = b / (uint32_t)(a.G * chunks);
    const uint32_t r = b - n * (uint32_t)(a.G * chunks);
    const uint32_t g = r / (uint32_t)chunks, ch = r - g * (uint32_t)chunks;
    const int WP = a.W + 2;                                  // bordered row
    const int plane = (a.H + 2) * WP;
    for (int i = threadIdx.x; i < plane * CC; i += blockDim.x) acc[i] = 0ull;

    const char* oimg = static_cast<const char*>(a.off) + (int64_t)n * a.img_off_elems * s;
    const char* mimg = static_cast<const char*>(a.msk) + (int64_t)n * a.img_mask_elems * s;
    const char* gimg = static_cast<const char*>(a.gout) + (int64_t)n * a.img_out_elems * s;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(oimg, a.img_off_bytes);
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(mimg, a.img_mask_bytes);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(gimg, a.img_out_bytes);
    const int npix = a.Ho * a.Wo;

    // ---- the scale: max|m| and max|g| over the (image, group); a non-finite
    // value (which a maximum would skip for NaN) is flagged on its own
    float mm = 0.0f, mg = 0.0f;
    bool bad = false;
    for (int pix = threadIdx.x; pix < npix; pix += blockDim.x) {
        RowLoad<DT, P> mrow;
        mrow.load(rm, (uint32_t)(((int64_t)pix * a.mask_row + (int64_t)g * P) * s));
#pragma unroll
        for (int k = 0; k < P; ++k) {
            const float v = mrow.get(k);
            mm = fmaxf(mm, fabsf(v));
            bad |= !isfinite(v);
        }
        const uint32_t gstart = (uint32_t)(((int64_t)pix * a.C + (int64_t)g * a.Cg) * s);
        for (int c0 = 0; c0 < a.Cg; c0 += 16) {
            RowLoad<DT, 16> gl;
            gl.load(rg, gstart + (uint32_t)(c0 * s));
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                if (c0 + c < a.Cg) {
                    const float v = gl.get(c);
                    mg = fmaxf(mg, fabsf(v));
                    bad |= !isfinite(v);
                }
            }
        }
    }
    for (int off = 32; off >= 1; off >>= 1) {
        mm = fmaxf(mm, __shfl_xor(mm, off));
        mg = fmaxf(mg, __shfl_xor(mg, off));
    }
    const bool wave_bad = __any(bad);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { red[0][wave] = mm; red[1][wave] = mg; flag[wave] = wave_bad; }
    __syncthreads();
    mm = 0.0f; mg = 0.0f;
    bool fixed = true;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
        mm = fmaxf(mm, red[0][w]);
        mg = fmaxf(mg, red[1][w]);
        fixed = fixed & !flag[w];
    }
    const float M = mm * mg;
    fixed = fixed & isfinite(M);
    int F = 0;
    if (fixed && M > 0.0f) {
        int e;
        frexpf(M, &e);                        // M < 2^e
        // sums below 2^62, and each term below 2^51 (for the conversion below)
        F = (a.cbits < 11 ? 51 : 62 - a.cbits) - e;
    }

    const double scaleF = ldexp(1.0, F);
    const float fW = (float)a.W, fH = (float)a.H;
    float* accf = reinterpret_cast<float*>(acc);
    for (int it = threadIdx.x; it < npix; it += blockDim.x) {
        const int pix = spread_index(it, npix);
        const int ho = pix / a.Wo, wo = pix - (pix / a.Wo) * a.Wo;
        // the unit's offset, weight and output-gradient rows: all loads in flight together
        RowLoad<DT, 2 * P> orow;
        RowLoad<DT, P> mrow;
        RowLoad<DT, CC> grow;
        orow.load(ro, (uint32_t)(((int64_t)pix * a.off_row + (int64_t)g * 2 * P) * s));
        mrow.load(rm, (uint32_t)(((int64_t)pix * a.mask_row + (int64_t)g * P) * s));
        grow.load(rg, (uint32_t)(((int64_t)pix * a.C + (int64_t)g * a.Cg + (int64_t)ch * CC) * s));
        float gr[CC];
        double gd[CC];
#pragma unroll
        for (int c = 0; c < CC; ++c) {
            gr[c] = grow.get(c);
            gd[c] = (double)gr[c];
        }
        const int bx0 = wo * a.stride - a.pad, by0 = ho * a.stride - a.pad;
#pragma unroll
        for (int k = 0; k < P; ++k) {
            const int q = (RC && k >= 4) ? k + 1 : k;
            const int i = q / 3, j = q % 3;
            const float px = fmaf(orow.get(k), a.offset_scale, (float)(bx0 + j * a.dil));
            const float py = fmaf(orow.get(P + k), a.offset_scale, (float)(by0 + i * a.dil));
            const float m = mrow.get(k);
            if (!((px > -1.0f) & (px < fW) & (py > -1.0f) & (py < fH))) continue;
            const float fx = floorf(px), fy = floorf(py);
            const int x0 = (int)fx, y0 = (int)fy;
            const float lx = px - fx, ly = py - fy;
            const float hx = 1.0f - lx, hy = 1.0f - ly;
            const float mhy = m * hy, mly = m * ly;
            const float w[4] = {mhy * hx, mhy * lx, mly * hx, mly * lx};
            const int cell[4] = {0, 1, WP, WP + 1};
            // corner (y0, x0) of the bordered image; the others follow
            const int c00 = (y0 + 1) * WP + (x0 + 1);
            if (fixed) {
                // term w * g on the grid of 2^-F: the product of the binary32
                // factors is exact in binary64 (w pre-scaled by 2^F, exactly),
                // |product| < 2^51.  Adding 1.5 * 2^52 rounds it to the
                // nearest integer q (ties to even) and leaves q + 2^51 in the
                // low 52 bits of the sum's pattern, whose high 12 bits are
                // those of 1.5 * 2^52: the pattern minus that of 1.5 * 2^52
                // is q as a two's-complement 64-bit integer
                constexpr double kMagic = 0x1.8p52;
                constexpr unsigned long long kMagicBits = 0x4338000000000000ull;
                double wd[4];
#pragma unroll
                for (int cr = 0; cr < 4; ++cr) wd[cr] = (double)w[cr] * scaleF;
#pragma unroll
                for (int cr = 0; cr < 4; ++cr) {
#pragma unroll
                    for (int c = 0; c < CC; ++c) {
                        const double t = wd[cr] * gd[c] + kMagic;
                        const unsigned long long u = __double_as_longlong(t) - kMagicBits;
                        atomicAdd(&acc[c * plane + c00 + cell[cr]], u);
                    }
                }
            } else {
#pragma unroll
                for (int cr = 0; cr < 4; ++cr) {
#pragma unroll
                    for (int c = 0; c < CC; ++c) atomicAdd(&accf[c * plane + c00 + cell[cr]], w[cr] * gr[c]);
                }
            }
        }
    }
    __syncthreads();

    // the image's interior to grad_x[n, y, x, g*Cg + ch*CC + c]
    float* gx = a.gx + (int64_t)n * a.img_x_elems + g * a.Cg + ch * CC;
    const int interior = a.H * a.W * CC;
    for (int i = threadIdx.x; i < interior; i += blockDim.x) {
        const int c = i % CC, p = i / CC;
        const int y = p / a.W, x = p - (p / a.W) * a.W;
        const int idx = c * plane + (y + 1) * WP + (x + 1);
        gx[(int64_t)p * a.C + c] = fixed ? (float)ldexp((double)(long long)acc[idx], -F) : accf[idx];
    }
}

// First output index along one axis whose clamped grid centre
// min(max(o * stride + c0, 0), in - 1) is at least lim (`outs` if none).
__device__ __forceinline__ int first_output(int lim, int c0, int stride, int in, int outs)
{
    if (lim <= 0) return 0;
    if (lim > in - 1) return outs;
    const int d = lim - c0;
    const int o = d >= 0 ? (d + stride - 1) / stride : -((-d) / stride);
    return min(max(o, 0), outs);
}

// x's gradient of one (image, group, chunk of CC channels, tile of TS x TS
// pixels), for images whose bordered plane does not fit in LDS.  A unit's
// centre is the middle point of its sampling grid, clamped into the image;
// its home tile holds the centre.  The workgroup visits the units whose
// centre lies within `margin` pixels of its tile and accumulates, in an LDS
// copy of the tile (64-bit fixed point as above, F per workgroup from the
// units it visits), the terms of their corners inside the tile.  A corner in
// another tile is that tile's when its workgroup visits the unit too; if not,
// the unit's home workgroup adds the term to grad_x with a global binary32
// atomic add.  Each term is added once.  grad_x is zeroed beforehand and every
// tile adds its sums with atomic adds as well (global terms from other tiles
// may land on the same elements): an element without global terms is exactly
// its fixed-point sum, rounded once; the others are summed in no fixed order.
template <int DT, int RC, int CC>
__global__ void __launch_bounds__(1024) k_backward_x_tiled(BArgs a, uint32_t total_blocks, uint32_t per_xcd)
{
    using E = Elem<DT>;
    constexpr int s = E::kBytes;
    constexpr int P = 9 - RC;                 // K = 3
    extern __shared__ unsigned long long acc[];
    __shared__ BxShared sh_;
    float (&red)[2][16] = sh_.red;
    bool (&flag)[16] = sh_.flag;
    const int chunks = a.Cg / CC;
    uint32_t b;
    if (!logical_block(blockIdx.x, total_blocks, per_xcd, &b)) return;
    // b = ((n * tiles + t) * G + g) * chunks + ch: the groups and chunks of a
    // tile, which read the same offset and weight rows, on one XCD
    const uint32_t gc = (uint32_t)(a.G * chunks);
    const uint32_t nt = b / gc, r = b - nt * gc;
    const uint32_t ntiles = (uint32_t)(a.tiles_y * a.tiles_x);
    const uint32_t n = nt / ntiles, t = nt - n * ntiles;
    const uint32_t g = r / (uint32_t)chunks, ch = r - g * (uint32_t)chunks;
    const int sh = a.tile_sh, TS = 1 << sh, TP = TS * TS;
    const int tyi = (int)t / a.tiles_x, txi = (int)t - tyi * a.tiles_x;
    const int ty0 = tyi << sh, tx0 = txi << sh;
    const int th = min(TS, a.H - ty0), tw = min(TS, a.W - tx0);
    for (int i = threadIdx.x; i < TP * CC; i += blockDim.x) acc[i] = 0ull;

    // the visited units: output rectangle [hlo, hhi) x [wlo, whi)
    const int M = a.margin;
    const int c0 = a.dil - a.pad;             // grid centre of output 0
    const int hlo = first_output(ty0 - M, c0, a.stride, a.H, a.Ho);
    const int hhi = max(hlo, first_output(ty0 + TS + M, c0, a.stride, a.H, a.Ho));
    const int wlo = first_output(tx0 - M, c0, a.stride, a.W, a.Wo);
    const int whi = max(wlo, first_output(tx0 + TS + M, c0, a.stride, a.W, a.Wo));
    const int wcnt = whi - wlo;
    const int nunits = (hhi - hlo) * wcnt;

    const char* oimg = static_cast<const char*>(a.off) + (int64_t)n * a.img_off_elems * s;
    const char* mimg = static_cast<const char*>(a.msk) + (int64_t)n * a.img_mask_elems * s;
    const char* gimg = static_cast<const char*>(a.gout) + (int64_t)n * a.img_out_elems * s;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(oimg, a.img_off_bytes);
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(mimg, a.img_mask_bytes);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(gimg, a.img_out_bytes);
    const int64_t chan0 = (int64_t)g * a.Cg + (int64_t)ch * CC;

    // ---- the scale: max|m| and max|g| over the visited units and the chunk
    float mm = 0.0f, mg = 0.0f;
    bool bad = false;
    for (int i = threadIdx.x; i < nunits; i += blockDim.x) {
        const int hh = i / wcnt;
        const int pix = (hlo + hh) * a.Wo + wlo + (i - hh * wcnt);
        RowLoad<DT, P> mrow;
        RowLoad<DT, CC> grow;
        mrow.load(rm, (uint32_t)(((int64_t)pix * a.mask_row + (int64_t)g * P) * s));
        grow.load(rg, (uint32_t)(((int64_t)pix * a.C + chan0) * s));
#pragma unroll
        for (int k = 0; k < P; ++k) {
            const float v = mrow.get(k);
            mm = fmaxf(mm, fabsf(v));
            bad |= !isfinite(v);
        }
#pragma unroll
        for (int c = 0; c < CC; ++c) {
            const float v = grow.get(c);
            mg = fmaxf(mg, fabsf(v));
            bad |= !isfinite(v);
        }
    }
    for (int off = 32; off >= 1; off >>= 1) {
        mm = fmaxf(mm, __shfl_xor(mm, off));
        mg = fmaxf(mg, __shfl_xor(mg, off));
    }
    const bool wave_bad = __any(bad);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { red[0][wave] = mm; red[1][wave] = mg; flag[wave] = wave_bad; }
    __syncthreads();
    mm = 0.0f; mg = 0.0f;
    bool fixed = true;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
        mm = fmaxf(mm, red[0][w]);
        mg = fmaxf(mg, red[1][w]);
        fixed = fixed & !flag[w];
    }
    const float Mv = mm * mg;
    fixed = fixed & isfinite(Mv);
    int F = 0;
    if (fixed && Mv > 0.0f) {
        // terms per element: at most (visited units) * P points * 4 corners
        const int64_t terms = (int64_t)nunits * P * 4;
        int cbits = 0;
        while (((int64_t)1 << cbits) < terms) ++cbits;
        int e;
        frexpf(Mv, &e);                       // Mv < 2^e
        F = (cbits < 11 ? 51 : 62 - cbits) - e;
    }

    const double scaleF = ldexp(1.0, F);
    const float fW = (float)a.W, fH = (float)a.H;
    float* accf = reinterpret_cast<float*>(acc);
    float* gxi = a.gx + (int64_t)n * a.img_x_elems + chan0;
    for (int i = threadIdx.x; i < nunits; i += blockDim.x) {
        const int hh = i / wcnt;
        const int ho = hlo + hh, wo = wlo + (i - hh * wcnt);
        const int pix = ho * a.Wo + wo;
        RowLoad<DT, 2 * P> orow;
        RowLoad<DT, P> mrow;
        RowLoad<DT, CC> grow;
        orow.load(ro, (uint32_t)(((int64_t)pix * a.off_row + (int64_t)g * 2 * P) * s));
        mrow.load(rm, (uint32_t)(((int64_t)pix * a.mask_row + (int64_t)g * P) * s));
        grow.load(rg, (uint32_t)(((int64_t)pix * a.C + chan0) * s));
        float gr[CC];
        double gd[CC];
#pragma unroll
        for (int c = 0; c < CC; ++c) {
            gr[c] = grow.get(c);
            gd[c] = (double)gr[c];
        }
        const int cy = min(max(ho * a.stride + c0, 0), a.H - 1);
        const int cx = min(max(wo * a.stride + c0, 0), a.W - 1);
        const bool home = (cy >> sh) == tyi && (cx >> sh) == txi;
        const int bx0 = wo * a.stride - a.pad, by0 = ho * a.stride - a.pad;
#pragma unroll
        for (int k = 0; k < P; ++k) {
            const int q = (RC && k >= 4) ? k + 1 : k;
            const int i3 = q / 3, j3 = q % 3;
            const float px = fmaf(orow.get(k), a.offset_scale, (float)(bx0 + j3 * a.dil));
            const float py = fmaf(orow.get(P + k), a.offset_scale, (float)(by0 + i3 * a.dil));
            const float m = mrow.get(k);
            if (!((px > -1.0f) & (px < fW) & (py > -1.0f) & (py < fH))) continue;
            const float fx = floorf(px), fy = floorf(py);
            const int x0 = (int)fx, y0 = (int)fy;
            const float lx = px - fx, ly = py - fy;
            const float hx = 1.0f - lx, hy = 1.0f - ly;
            const float mhy = m * hy, mly = m * ly;
            const float w[4] = {mhy * hx, mhy * lx, mly * hx, mly * lx};
            const int ry = y0 - ty0, rx = x0 - tx0;
            const bool iny[2] = {(unsigned)ry < (unsigned)th, (unsigned)(ry + 1) < (unsigned)th};
            const bool inx[2] = {(unsigned)rx < (unsigned)tw, (unsigned)(rx + 1) < (unsigned)tw};
#pragma unroll
            for (int cr = 0; cr < 4; ++cr) {
                const int dy = cr >> 1, dx = cr & 1;
                if (iny[dy] & inx[dx]) {
                    const int cell = (ry + dy) * TS + rx + dx;
                    if (fixed) {
                        // the exact term rounded to the grid of 2^-F, as in k_backward_x
                        constexpr double kMagic = 0x1.8p52;
                        constexpr unsigned long long kMagicBits = 0x4338000000000000ull;
                        const double wd = (double)w[cr] * scaleF;
#pragma unroll
                        for (int c = 0; c < CC; ++c) {
                            const double tv = wd * gd[c] + kMagic;
                            atomicAdd(&acc[c * TP + cell], (unsigned long long)__double_as_longlong(tv) - kMagicBits);
                        }
                    } else {
#pragma unroll
                        for (int c = 0; c < CC; ++c) atomicAdd(&accf[c * TP + cell], w[cr] * gr[c]);
                    }
                } else if (home) {
                    const int qy = y0 + dy, qx = x0 + dx;
                    // the corner's tile visits this unit iff the centre is within its margin
                    const bool reached = (unsigned)(cy - ((qy >> sh) << sh) + M) < (unsigned)(TS + 2 * M) &&
                                         (unsigned)(cx - ((qx >> sh) << sh) + M) < (unsigned)(TS + 2 * M);
                    if ((unsigned)qy < (unsigned)a.H && (unsigned)qx < (unsigned)a.W && !reached) {
                        float* dst = gxi + ((int64_t)qy * a.W + qx) * a.C;
#pragma unroll
                        for (int c = 0; c < CC; ++c) unsafeAtomicAdd(dst + c, w[cr] * gr[c]);
                    }
                }
            }
        }
    }
    __syncthreads();

    // the tile's sums into grad_x[n, y, x, g*Cg + ch*CC + c]
    const int cells = th * tw * CC;
    for (int i = threadIdx.x; i < cells; i += blockDim.x) {
        const int c = i % CC, p = i / CC;
        const int yy = p / tw, xx = p - (p / tw) * tw;
        const int idx = c * TP + yy * TS + xx;
        const float v = fixed ? (float)ldexp((double)(long long)acc[idx], -F) : accf[idx];
        unsafeAtomicAdd(gxi + ((int64_t)(ty0 + yy) * a.W + tx0 + xx) * a.C + c, v);
    }
}

template <int DT, int RC>
void launch_bxt_cc(const BArgs& a, unsigned total, size_t lds, hipStream_t stream)
{
    const uint32_t per_xcd = (total + 7) / 8;
    const unsigned grid = per_xcd * 8;
    switch (a.cc) {
        case 16: hipLaunchKernelGGL((k_backward_x_tiled<DT, RC, 16>), dim3(grid), dim3(1024), lds, stream, a, total, per_xcd); break;
        case 8: hipLaunchKernelGGL((k_backward_x_tiled<DT, RC, 8>), dim3(grid), dim3(1024), lds, stream, a, total, per_xcd); break;
        case 4: hipLaunchKernelGGL((k_backward_x_tiled<DT, RC, 4>), dim3(grid), dim3(1024), lds, stream, a, total, per_xcd); break;
        case 2: hipLaunchKernelGGL((k_backward_x_tiled<DT, RC, 2>), dim3(grid), dim3(1024), lds, stream, a, total, per_xcd); break;
        default: hipLaunchKernelGGL((k_backward_x_tiled<DT, RC, 1>), dim3(grid), dim3(1024), lds, stream, a, total, per_xcd); break;
    }
}

template <int DT>
void launch_bxt(const BArgs& a, unsigned grid, size_t lds, hipStream_t stream)
{
    if (a.remove_center) launch_bxt_cc<DT, 1>(a, grid, lds, stream);
    else launch_bxt_cc<DT, 0>(a, grid, lds, stream);
}

template <int DT, int RC>
void launch_bx_cc(const BArgs& a, unsigned total, size_t lds, hipStream_t stream)
{
    const uint32_t per_xcd = (total + 7) / 8;
    const unsigned grid = per_xcd * 8;
    switch (a.cc) {
        case 16: hipLaunchKernelGGL((k_backward_x<DT, RC, 16>), dim3(grid), dim3(1024), lds, stream, a, total, per_xcd); break;
        case 8: hipLaunchKernelGGL((k_backward_x<DT, RC, 8>), dim3(grid), dim3(1024), lds, stream, a, total, per_xcd); break;
        case 4: hipLaunchKernelGGL((k_backward_x<DT, RC, 4>), dim3(grid), dim3(1024), lds, stream, a, total, per_xcd); break;
        case 2: hipLaunchKernelGGL((k_backward_x<DT, RC, 2>), dim3(grid), dim3(1024), lds, stream, a, total, per_xcd); break;
        default: hipLaunchKernelGGL((k_backward_x<DT, RC, 1>), dim3(grid), dim3(1024), lds, stream, a, total, per_xcd); break;
    }
}

template <int DT>
void launch_bx(const BArgs& a, unsigned grid, size_t lds, hipStream_t stream)
{
    if (a.remove_center) launch_bx_cc<DT, 1>(a, grid, lds, stream);
    else launch_bx_cc<DT, 0>(a, grid, lds, stream);
}

template <int DT, int VB>
void launch_vb(const BArgs& a, int64_t grid, hipStream_t stream)
{
    // each XCD a contiguous range of blocks when an image fits in its L2 (4 MB)
    const uint32_t total = (uint32_t)grid;
    const uint32_t per_xcd = a.img_x_bytes <= (4u << 20) ? (total + 7) / 8 : 0u;
    const uint32_t launched = per_xcd ? per_xcd * 8 : total;
    if (a.K == 3)
        hipLaunchKernelGGL((k_backward<DT, VB, 3>), dim3(launched), dim3(256), 0, stream, a, total, per_xcd);
    else
        hipLaunchKernelGGL((k_backward<DT, VB, 0>), dim3(launched), dim3(256), 0, stream, a, total, per_xcd);
}

template <int DT>
hipError_t launch_dt(const BArgs& a, int64_t grid, hipStream_t stream)
{
    switch (a.vec_bytes) {
        case 16: launch_vb<DT, 16>(a, grid, stream); break;
        case 8: launch_vb<DT, 8>(a, grid, stream); break;
        case 4: launch_vb<DT, 4>(a, grid, stream); break;
        case 2:
            if constexpr (DT != DCNV4_F32) {
                launch_vb<DT, 2>(a, grid, stream);
                break;
            }
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

int backward_vec_bytes(const Problem& p, const void* gout)
{
    const int s = p.dtype == DCNV4_F32 ? 4 : 2;
    int vb = 16;
    while (vb > s) {
        if ((p.Cg * s) % vb == 0 && (uintptr_t)p.x % vb == 0 && (uintptr_t)gout % vb == 0) break;
        vb >>= 1;
    }
    return vb;
}

void plan_backward(const Problem& p, const void* gout, bool want_x, bool want_om, BwdPlan* bp)
{
    memset(bp, 0, sizeof *bp);
    // x's gradient in LDS when a channel chunk of the bordered image fits,
    // else in LDS tiles (K = 3), else with global atomics only
    int cc = want_x ? backward_x_chunk(p) : 0;
    // one workgroup per (image, group, chunk) holds a CU for the whole
    // image: with at most a quarter as many of them as CUs (small batches),
    // tiles fill the GPU.  Tiles add visits of the units around them, which
    // measured slower than the whole image with a third of the CUs busy (the
    // latent shape at batch 1: 103 against 94 us) and faster with a quarter
    // (stage-1 shape at batch 4: 50 against 62 us)
    if (cc && backward_fill_gpu() && (int64_t)p.N * p.G * (p.Cg / cc) * 4 <= p.cus) cc = 0;
    if (!want_x) {
        bp->x_path = 0;
    } else if (cc) {
        bp->x_path = 1;
        bp->cc = cc;
        bp->x_lds = (int)((int64_t)(p.H + 2) * (p.W + 2) * cc * 8) + kBwdXStaticLds;
    } else if (backward_x_tiles(p, &bp->cc, &bp->tile_sh, &bp->margin)) {
        bp->x_path = 2;
        bp->x_lds = (int)(((int64_t)1 << (2 * bp->tile_sh)) * bp->cc * 8) + kBwdXStaticLds;
    } else {
        bp->x_path = 3;
    }
    // offset and weight gradients from an LDS copy of each (image, group)
    // when it fits, unless x's gradient needs the atomics kernel anyway
    if (!want_om) bp->om_path = 0;
    else if (bp->x_path != 3 && backward_om_window_plan(p, gout, &bp->om)) bp->om_path = 1;
    else bp->om_path = 2;
}

hipError_t launch_backward(const Problem& p, const void* gout, float* gx, float* goff, float* gmask,
                           hipStream_t stream)
{
    const int s = p.dtype == DCNV4_F32 ? 4 : 2;
    BArgs a;
    memset(&a, 0, sizeof a);
    a.x = p.x; a.off = p.off; a.msk = p.msk; a.gout = gout;
    a.gx = gx; a.goff = goff; a.gmask = gmask;
    a.H = p.H; a.W = p.W; a.G = p.G; a.Cg = p.Cg; a.C = p.G * p.Cg;
    a.K = p.K; a.P = p.P; a.stride = p.stride; a.pad = p.pad; a.dil = p.dil;
    a.Ho = p.Ho; a.Wo = p.Wo; a.remove_center = p.remove_center;
    a.off_row = p.off_row; a.mask_row = p.mask_row;
    a.offset_scale = p.offset_scale;
    a.img_x_elems = (int64_t)p.H * p.W * a.C;
    a.img_out_elems = (int64_t)p.Ho * p.Wo * a.C;
    a.img_off_elems = (int64_t)p.Ho * p.Wo * p.off_row;
    a.img_mask_elems = (int64_t)p.Ho * p.Wo * p.mask_row;
    a.img_x_bytes = (uint32_t)(a.img_x_elems * s);
    a.img_out_bytes = (uint32_t)(a.img_out_elems * s);
    a.img_off_bytes = (uint32_t)(((((int64_t)p.Ho * p.Wo - 1) * p.off_row + (int64_t)p.G * 2 * p.P) * s + 3) & ~3ll);
    a.img_mask_bytes = (uint32_t)(((((int64_t)p.Ho * p.Wo - 1) * p.mask_row + (int64_t)p.G * p.P) * s + 3) & ~3ll);
    a.vec_bytes = backward_vec_bytes(p, gout);
    a.lanes = p.Cg * s / a.vec_bytes;
    a.units_per_wave = 64 / a.lanes;
    a.units_img = (uint32_t)((int64_t)p.Ho * p.Wo * p.G);
    a.units_total = (int64_t)p.N * a.units_img;
    a.div_units_img = make_fastdiv(a.units_img);
    a.div_G = make_fastdiv((uint32_t)p.G);
    a.div_Wo = make_fastdiv((uint32_t)p.Wo);

    BwdPlan bp;
    plan_backward(p, gout, gx != nullptr, goff || gmask, &bp);
    const bool whole = bp.x_path == 1, tiled = bp.x_path == 2;
    a.cc = bp.cc;
    a.tile_sh = bp.tile_sh;
    a.margin = bp.margin;
    if (tiled) {
        a.tiles_y = (p.H + (1 << a.tile_sh) - 1) >> a.tile_sh;
        a.tiles_x = (p.W + (1 << a.tile_sh) - 1) >> a.tile_sh;
    }
    if (gx && !whole) {
        const int64_t n = (int64_t)p.N * a.img_x_elems;
        const int64_t blocks = ceil_div(ceil_div(n, 4), 256);
        hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0, stream, gx, n);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const bool om_window = bp.om_path == 1;
    if (om_window) {
        const OmPlan& om = bp.om;
        BArgs b = a;
        b.gx = nullptr;
        b.pitch = om.pitch;
        b.om_th = om.th; b.om_tw = om.tw; b.om_ry = om.ry; b.om_rx = om.rx;
        b.om_wh = om.wh; b.om_ww = om.ww; b.om_tiles_y = om.tiles_y; b.om_tiles_x = om.tiles_x;
        b.div_om_tw = make_fastdiv((uint32_t)om.tw);
        const hipError_t e = launch_backward_om_window(b, p.dtype, p.Cg * s / 16, om.block, om.lds, stream);
        if (e != hipSuccess) return e;
    }
    if ((!om_window && (goff || gmask)) || (gx && !whole && !tiled)) {
        BArgs b = a;
        if (whole || tiled) b.gx = nullptr;   // an LDS kernel below takes x's gradient
        if (om_window) b.goff = b.gmask = nullptr;
        const int64_t grid = ceil_div(a.units_total, 4 * (int64_t)a.units_per_wave);
        hipError_t e = hipErrorInvalidValue;
        switch (p.dtype) {
            case DCNV4_F32: e = launch_dt<DCNV4_F32>(b, grid, stream); break;
            case DCNV4_F16: e = launch_dt<DCNV4_F16>(b, grid, stream); break;
            case DCNV4_BF16: e = launch_dt<DCNV4_BF16>(b, grid, stream); break;
            default: break;
        }
        if (e != hipSuccess) return e;
    }
    if (tiled) {
        const unsigned grid = (unsigned)((int64_t)p.N * a.tiles_y * a.tiles_x * p.G * (p.Cg / a.cc));
        const size_t lds = ((size_t)1 << (2 * a.tile_sh)) * a.cc * 8;
        switch (p.dtype) {
            case DCNV4_F32: launch_bxt<DCNV4_F32>(a, grid, lds, stream); break;
            case DCNV4_F16: launch_bxt<DCNV4_F16>(a, grid, lds, stream); break;
            case DCNV4_BF16: launch_bxt<DCNV4_BF16>(a, grid, lds, stream); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if (whole) {
        // terms per x element: at most (units of the image) * P points * 4 corners
        const int64_t terms = (int64_t)p.Ho * p.Wo * p.P * 4;
        int cb = 0;
        while (((int64_t)1 << cb) < terms) ++cb;
        a.cbits = cb;
        const unsigned grid = (unsigned)((int64_t)p.N * p.G * (p.Cg / a.cc));
        const size_t lds = (size_t)(p.H + 2) * (p.W + 2) * a.cc * 8;
        switch (p.dtype) {
            case DCNV4_F32: launch_bx<DCNV4_F32>(a, grid, lds, stream); break;
            case DCNV4_F16: launch_bx<DCNV4_F16>(a, grid, lds, stream); break;
            case DCNV4_BF16: launch_bx<DCNV4_BF16>(a, grid, lds, stream); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    return hipSuccess;
}

bool backward_x_tiles(const Problem& p, int* cc, int* tile_sh, int* margin)
{
    // K = 3: tiles of 64 x 64 pixels, the most channels per workgroup (a
    // power of two dividing Cg, at most 16) whose tile of 64-bit accumulators
    // fits in LDS, and the units of a 16-pixel margin around the tile.  The
    // margin trades visits against global atomic adds: with offsets of 8
    // pixels' spread (256 x 256 images) 16 pixels measured fastest, ahead of
    // 12 (atomic adds) and 20 or more (visits)
    if (p.K != 3) return false;
    // the largest side from 64 down to 8 whose grid fills the GPU (8 if none does)
    int sh = 6, m = 16;
    if (backward_fill_gpu()) {
        for (; sh > 3; --sh) {
            int c = 16;
            while (c > 1 && (p.Cg % c || ((int64_t)8 << (2 * sh)) * c + kBwdXStaticLds > kLdsPerCu)) c /= 2;
            const int64_t tiles = (int64_t)((p.H + (1 << sh) - 1) >> sh) * ((p.W + (1 << sh) - 1) >> sh);
            if ((int64_t)p.N * tiles * p.G * (p.Cg / c) >= p.cus) break;
        }
    }
    // DCNV4_BWD_TILE="<log2 side>,<margin>" overrides both (side 8 to 128, margin 0 to 256)
    if (const char* env = getenv("DCNV4_BWD_TILE")) {
        int es = 0, em = 0;
        if (sscanf(env, "%d,%d", &es, &em) == 2 && es >= 3 && es <= 7 && em >= 0 && em <= 256) {
            sh = es;
            m = em;
        }
    }
    const int64_t cell = ((int64_t)1 << (2 * sh)) * 8;
    for (int c = 16; c >= 1; c /= 2) {
        if (p.Cg % c == 0 && cell * c + kBwdXStaticLds <= kLdsPerCu) {
            *cc = c;
            *tile_sh = sh;
            *margin = m;
            return true;
        }
    }
    return false;
}

bool backward_fill_gpu()
{
    // DCNV4_BWD_FILL=0 keeps the whole-image kernels whenever they fit (tests)
    const char* env = getenv("DCNV4_BWD_FILL");
    return !(env && env[0] == '0' && env[1] == '\0');
}

int backward_x_chunk(const Problem& p)
{
    // K = 3: the most channels (a power of two dividing Cg, at most 16) whose
    // bordered image of 64-bit accumulators fits in LDS beside the kernel's
    // static LDS
    if (p.K != 3) return 0;
    const int64_t cell = (int64_t)(p.H + 2) * (p.W + 2) * 8;
    for (int cc = 16; cc >= 1; cc /= 2)
        if (p.Cg % cc == 0 && cell * cc + kBwdXStaticLds <= kLdsPerCu) return cc;
    return 0;
}

}  // namespace dcnv4

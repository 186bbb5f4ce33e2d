// DCNv4 spatial-aggregation forward: gfx950 kernels.
//
// Operation: jsqmd.com/news/933833 ("不只是卷积的平替：我把DCNv4塞进Stable
// Diffusion的U-Net里"), section 1, code example "DCNv4核心计算流程示例": per output
// pixel and group, K*K points on the grid plus learned offsets, bilinear
// samples of the channels-last input (zero outside the image), each times a raw
// dynamic weight (no softmax: same section's first optimisation; bqwf.cn/news/
// 1148139 section 2.1), summed over the points.  Sampling, interpolation and
// aggregation are one kernel with no intermediate in memory (jsqmd.com/news/
// 933833 section 4, kernel fusion).
//
// The binary32 operation order is fixed (see include/dcnv4.h) and every kernel
// here follows it exactly, so results are bit-identical across kernels, vector
// widths and launch shapes.  Contraction is off for the whole file: the only
// fused multiply-adds are the explicit fmaf calls.

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "dcnv4.h"
#include "dcnv4_internal.h"

#pragma clang fp contract(off)

namespace dcnv4 {
namespace {

// ---------------------------------------------------------------------------
// I/O element types
// ---------------------------------------------------------------------------

template <int DT> struct Elem;

template <> struct Elem<DCNV4_F32> {
    using S = float;
    static __device__ __forceinline__ float to_f(S v) { return v; }
    static __device__ __forceinline__ S from_f(float f) { return f; }
};

template <> struct Elem<DCNV4_F16> {
    using S = _Float16;
    static __device__ __forceinline__ float to_f(S v) { return (float)v; }   // exact
    static __device__ __forceinline__ S from_f(float f) { return (S)f; }     // RNE
};

template <> struct Elem<DCNV4_BF16> {
    using S = uint16_t;
    static __device__ __forceinline__ float to_f(S v) {                     // exact
        return __uint_as_float((uint32_t)v << 16);
    }
    static __device__ __forceinline__ S from_f(float f) {                   // RNE
        uint32_t u = __float_as_uint(f);
        if ((u & 0x7fffffffu) > 0x7f800000u) return (S)((u >> 16) | 0x40u);  // quiet NaN
        u += 0x7fffu + ((u >> 16) & 1u);
        return (S)(u >> 16);
    }
};

// VEC consecutive elements, loaded and stored as one access.
template <typename S, int VEC>
struct alignas(sizeof(S) * VEC) Vec {
    S v[VEC];
};

struct Args {
    const void* x;
    const void* off;
    const void* msk;
    void* out;
    int H, W, G, Cg, C, K, P, stride, pad, dil, Ho, Wo;
    int remove_center;
    int lanes;              // lanes per unit = Cg / VEC
    int64_t off_row, mask_row;
    int64_t img_x;          // elements of one input image
    int64_t total;          // units * lanes
    float offset_scale;
};

// ---------------------------------------------------------------------------
// Kernel family 1: one lane per (unit, VEC channels).
//
// unit = (n, ho, wo, g).  Each lane recomputes its unit's sampling positions
// and bilinear weights for every point, gathers VEC channels at each of the
// four corners as one vector load, and accumulates in binary32 registers.
// ---------------------------------------------------------------------------

template <int DT, int VEC, int KT>
__global__ void __launch_bounds__(256)
k_gather_vec(Args a)
{
    using E = Elem<DT>;
    using S = typename E::S;
    using V = Vec<S, VEC>;

    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= a.total) return;
    const int lane_in_unit = (int)(t % a.lanes);
    const int64_t unit = t / a.lanes;
    const int g = (int)(unit % a.G);
    const int64_t pix = unit / a.G;
    const int wo = (int)(pix % a.Wo);
    const int64_t nh = pix / a.Wo;
    const int ho = (int)(nh % a.Ho);
    const int n = (int)(nh / a.Ho);

    const int K = KT > 0 ? KT : a.K;
    const int P = KT > 0 ? (KT * KT - a.remove_center) : a.P;
    const int center = (K * K) / 2;
    const S* xs = static_cast<const S*>(a.x) + (int64_t)n * a.img_x + g * a.Cg + lane_in_unit * VEC;
    const S* os = static_cast<const S*>(a.off) + pix * a.off_row + (int64_t)g * 2 * P;
    const S* ms = static_cast<const S*>(a.msk) + pix * a.mask_row + (int64_t)g * P;

    float acc[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) acc[c] = 0.0f;

    const float fW = (float)a.W, fH = (float)a.H;
    const int bx0 = wo * a.stride - a.pad;
    const int by0 = ho * a.stride - a.pad;

    const int KK = K * K;
    constexpr int kUnroll = KT > 0 ? KT * KT : 1;
#pragma unroll kUnroll
    for (int q = 0; q < (KT > 0 ? KT * KT : KK); ++q) {          // grid index q = i*K + j
        if (a.remove_center && q == center) continue;
        const int k = (a.remove_center && q > center) ? q - 1 : q;  // point index
        const int i = q / K, j = q - (q / K) * K;
        const float dx = E::to_f(os[k]);
        const float dy = E::to_f(os[P + k]);
        const float m = E::to_f(ms[k]);
        const float px = fmaf(dx, a.offset_scale, (float)(bx0 + j * a.dil));
        const float py = fmaf(dy, a.offset_scale, (float)(by0 + i * a.dil));
        if (!(px > -1.0f && px < fW && py > -1.0f && py < fH)) continue;
        const float fx = floorf(px), fy = floorf(py);
        const int x0 = (int)fx, y0 = (int)fy;
        const float lx = px - fx, ly = py - fy;
        const float hx = 1.0f - lx, hy = 1.0f - ly;
        const float mhy = m * hy, mly = m * ly;
        const float w00 = mhy * hx, w01 = mhy * lx, w10 = mly * hx, w11 = mly * lx;
        const bool iny0 = y0 >= 0, iny1 = y0 + 1 < a.H;
        const bool inx0 = x0 >= 0, inx1 = x0 + 1 < a.W;
        const int64_t r0 = ((int64_t)y0 * a.W + x0) * a.C;
        V v00, v01, v10, v11;
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
            v00.v[c] = E::from_f(0.0f); v01.v[c] = E::from_f(0.0f);
            v10.v[c] = E::from_f(0.0f); v11.v[c] = E::from_f(0.0f);
        }
        if (iny0 && inx0) v00 = *reinterpret_cast<const V*>(xs + r0);
        if (iny0 && inx1) v01 = *reinterpret_cast<const V*>(xs + r0 + a.C);
        if (iny1 && inx0) v10 = *reinterpret_cast<const V*>(xs + r0 + (int64_t)a.W * a.C);
        if (iny1 && inx1) v11 = *reinterpret_cast<const V*>(xs + r0 + (int64_t)a.W * a.C + a.C);
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
            float s = acc[c];
            s = fmaf(w00, E::to_f(v00.v[c]), s);
            s = fmaf(w01, E::to_f(v01.v[c]), s);
            s = fmaf(w10, E::to_f(v10.v[c]), s);
            s = fmaf(w11, E::to_f(v11.v[c]), s);
            acc[c] = s;
        }
    }

    V o;
#pragma unroll
    for (int c = 0; c < VEC; ++c) o.v[c] = E::from_f(acc[c]);
    S* outp = static_cast<S*>(a.out) + pix * (int64_t)a.C + g * a.Cg + lane_in_unit * VEC;
    *reinterpret_cast<V*>(outp) = o;
}

template <int DT, int VEC>
hipError_t launch_gather_vec(const Args& a, const Plan& plan, hipStream_t stream)
{
    dim3 grid((unsigned)plan.grid), block((unsigned)plan.block);
    if (a.K == 3)
        hipLaunchKernelGGL((k_gather_vec<DT, VEC, 3>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((k_gather_vec<DT, VEC, 0>), grid, block, 0, stream, a);
    return hipGetLastError();
}

template <int DT>
hipError_t dispatch_vec(const Args& a, const Plan& plan, hipStream_t stream)
{
    switch (plan.vec) {
        case 8: if constexpr (DT != DCNV4_F32) return launch_gather_vec<DT, 8>(a, plan, stream); break;
        case 4: return launch_gather_vec<DT, 4>(a, plan, stream);
        case 2: return launch_gather_vec<DT, 2>(a, plan, stream);
        case 1: return launch_gather_vec<DT, 1>(a, plan, stream);
        default: break;
    }
    return hipErrorInvalidValue;
}

}  // namespace

// ---------------------------------------------------------------------------
// Launch heuristics
// ---------------------------------------------------------------------------

void make_plan(const Problem& p, Plan* plan)
{
    const int s = p.dtype == DCNV4_F32 ? 4 : 2;
    // Widest vector (<= 16 bytes) that divides Cg and keeps every gather and
    // store aligned: x and out base pointers must be aligned to vec * s bytes;
    // channel offsets are multiples of vec because C = G*Cg and Cg % vec == 0.
    int vec = 16 / s;
    while (vec > 1) {
        const uintptr_t al = (uintptr_t)vec * s;
        if (p.Cg % vec == 0 && ((uintptr_t)p.x % al) == 0 && ((uintptr_t)p.out % al) == 0) break;
        vec >>= 1;
    }
    plan->kernel = kKernelGatherVec;
    plan->vec = vec;
    plan->lanes = p.Cg / vec;
    plan->block = 256;
    const int64_t units = (int64_t)p.N * p.Ho * p.Wo * p.G;
    const int64_t total = units * plan->lanes;
    plan->grid = (total + plan->block - 1) / plan->block;
}

hipError_t launch_forward(const Problem& p, const Plan& plan, hipStream_t stream)
{
    Args a;
    a.x = p.x; a.off = p.off; a.msk = p.msk; a.out = p.out;
    a.H = p.H; a.W = p.W; a.G = p.G; a.Cg = p.Cg; a.C = p.G * p.Cg;
    a.K = p.K; a.P = p.P; a.stride = p.stride; a.pad = p.pad; a.dil = p.dil;
    a.Ho = p.Ho; a.Wo = p.Wo; a.remove_center = p.remove_center;
    a.lanes = plan.lanes;
    a.off_row = p.off_row; a.mask_row = p.mask_row;
    a.img_x = (int64_t)p.H * p.W * a.C;
    a.total = (int64_t)p.N * p.Ho * p.Wo * p.G * plan.lanes;
    a.offset_scale = p.offset_scale;
    switch (p.dtype) {
        case DCNV4_F32: return dispatch_vec<DCNV4_F32>(a, plan, stream);
        case DCNV4_F16: return dispatch_vec<DCNV4_F16>(a, plan, stream);
        case DCNV4_BF16: return dispatch_vec<DCNV4_BF16>(a, plan, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dcnv4

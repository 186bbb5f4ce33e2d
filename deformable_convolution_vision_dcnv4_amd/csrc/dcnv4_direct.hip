// DCNv4 forward, "direct" kernel family: corner gathers straight from global
// memory.  The general path: any K, stride, pad, dilation, channel count,
// pointer alignment and offset/weight row stride.
//
// Operation: jsqmd.com/news/933833 ("不只是卷积的平替：我把DCNv4塞进Stable
// Diffusion的U-Net里"), section 1, code example "DCNv4核心计算流程示例": grid
// point + learned offset, bilinear sample with zero padding, times the raw
// dynamic weight, summed over the points; no softmax (same section, first
// optimisation; bqwf.cn/news/1148139 section 2.1).
//
// Layout of the work: a block covers 256 consecutive (unit, vector) lanes of
// ONE image, unit = (ho, wo, g), so every buffer resource is uniform across
// the block.  When an image fits in one XCD's L2 (4 MB), blocks are
// renumbered so that each XCD runs a contiguous range of them (whole images
// or bands of output rows): the corners its blocks gather then mostly stay
// in that XCD's L2 (measured 14-17% faster on the 56x56 and 14x14 shapes, 5%
// on the 64x64 latent).  Larger images keep the round-robin order, measured
// faster on the 256x256 shape with its long offsets.  Corner reads are raw buffer loads: a corner outside the image
// gets an out-of-range offset and reads zero, so the loads carry no branch and
// are all issued before the first multiply-add.

#include "dcnv4_device.h"
#include "dcnv4_kernels.h"

namespace dcnv4 {
namespace {

constexpr uint32_t kL2PerXcd = 4u << 20;

template <int VB>
__device__ __forceinline__ void load_corner(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t* d)
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

// acc[0..VB/s) += w * elements of d (little-endian element order).
template <int DT, int VB>
__device__ __forceinline__ void fma_raw(float* acc, float w, const uint32_t* d)
{
    using E = Elem<DT>;
    constexpr int n = VB / E::kBytes;
    if constexpr (DT == DCNV4_F32) {
#pragma unroll
        for (int i = 0; i < n; ++i) acc[i] = fmaf(w, __uint_as_float(d[i]), acc[i]);
    } else {
#pragma unroll
        for (int i = 0; i < n; ++i) {
            const uint32_t word = d[i / 2];
            const uint32_t half = (i & 1) ? (word >> 16) : (word & 0xffffu);
            acc[i] = fmaf(w, E::raw_to_f(half), acc[i]);
        }
    }
}

template <int DT, int VB>
__device__ __forceinline__ void store_raw(void* out, int64_t elem, const float* acc)
{
    using E = Elem<DT>;
    using S = typename E::S;
    constexpr int n = VB / E::kBytes;
    struct alignas(VB) V { S v[n]; };
    V o;
#pragma unroll
    for (int i = 0; i < n; ++i) o.v[i] = E::from_f(settle(acc[i]));
    *reinterpret_cast<V*>(static_cast<S*>(out) + elem) = o;
}

template <int DT, int VB, int KT, int SM>
__global__ void __launch_bounds__(256)
k_direct(KArgs a, uint32_t total_blocks, uint32_t per_xcd)
{
    using E = Elem<DT>;
    using S = typename E::S;
    constexpr int s = E::kBytes;
    constexpr int NE = VB / s;                 // elements per lane
    constexpr int NW = (VB + 3) / 4;           // dwords per corner read

    uint32_t lb = blockIdx.x;
    if (per_xcd && !logical_block(blockIdx.x, total_blocks, per_xcd, &lb)) return;
    const uint32_t n = lb / a.blocks_per_image;
    const uint32_t t = (lb - n * a.blocks_per_image) * 256u + threadIdx.x;
    const uint32_t unit = fdiv(t, a.div_lanes);
    if (unit >= a.units_img) return;
    const uint32_t lane_in_unit = t - unit * (uint32_t)a.lanes;
    const uint32_t pix = fdiv(unit, a.div_G);              // pixel within the image
    const uint32_t g = unit - pix * (uint32_t)a.G;
    const uint32_t ho = fdiv(pix, a.div_Wo);
    const uint32_t wo = pix - ho * (uint32_t)a.Wo;

    const int K = KT > 0 ? KT : a.K;
    const int P = a.P;
    const int center = (K * K) / 2;

    const S* xs = static_cast<const S*>(a.x) + (int64_t)n * a.img_x_elems;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(xs, a.img_x_bytes);
    const S* os = static_cast<const S*>(a.off) + (int64_t)n * a.img_off_elems + (int64_t)pix * a.off_row + g * 2 * P;
    const S* ms = static_cast<const S*>(a.msk) + (int64_t)n * a.img_mask_elems + (int64_t)pix * a.mask_row + g * P;
    const uint32_t chan_byte = (g * (uint32_t)a.Cg + lane_in_unit * NE) * s;
    const uint32_t pix_bytes = (uint32_t)a.C * s;
    const uint32_t row_bytes = (uint32_t)a.W * pix_bytes;

    float acc[NE];
#pragma unroll
    for (int c = 0; c < NE; ++c) acc[c] = 0.0f;

    // DCNv3-style weights (SM): w_k = exp(m_k - max) / sum_j exp(m_j - max),
    // the sum in point order, exp recomputed identically in the main loop
    float mx = 0.0f, rs = 0.0f;
    if (SM) {
        mx = E::to_f(ms[0]);
        for (int k = 1; k < P; ++k) mx = fmaxf(mx, E::to_f(ms[k]));
        for (int k = 0; k < P; ++k) rs += expf(E::to_f(ms[k]) - mx);
    }

    const float fW = (float)a.W, fH = (float)a.H;
    const int bx0 = (int)wo * a.stride - a.pad;
    const int by0 = (int)ho * a.stride - a.pad;
    constexpr int kUnroll = KT > 0 ? KT * KT : 1;
    const int KK = K * K;
#pragma unroll kUnroll
    for (int q = 0; q < (KT > 0 ? KT * KT : KK); ++q) {
        if (a.remove_center && q == center) continue;
        const int k = (a.remove_center && q > center) ? q - 1 : q;
        const int i = q / K, j = q - (q / K) * K;
        const float mk = SM ? expf(E::to_f(ms[k]) - mx) / rs : E::to_f(ms[k]);
        const PointCoef c = point_coef(E::to_f(os[k]), E::to_f(os[P + k]), mk,
                                       a.offset_scale, (float)(bx0 + j * a.dil), (float)(by0 + i * a.dil),
                                       fW, fH);
        // bitwise & and precomputed candidates: the corner reads carry no branch
        const bool iny0 = c.valid & (c.y0 >= 0), iny1 = c.valid & (c.y0 + 1 < a.H);
        const bool inx0 = c.x0 >= 0, inx1 = c.x0 + 1 < a.W;
        const uint32_t base = (uint32_t)c.y0 * row_bytes + (uint32_t)c.x0 * pix_bytes + chan_byte;
        const uint32_t b01 = base + pix_bytes, b10 = base + row_bytes, b11 = b10 + pix_bytes;
        const uint32_t o00 = (iny0 & inx0) ? base : kOobOffset;
        const uint32_t o01 = (iny0 & inx1) ? b01 : kOobOffset;
        const uint32_t o10 = (iny1 & inx0) ? b10 : kOobOffset;
        const uint32_t o11 = (iny1 & inx1) ? b11 : kOobOffset;
        uint32_t d00[NW], d01[NW], d10[NW], d11[NW];
        load_corner<VB>(rx, o00, d00);
        load_corner<VB>(rx, o01, d01);
        load_corner<VB>(rx, o10, d10);
        load_corner<VB>(rx, o11, d11);
        fma_raw<DT, VB>(acc, c.w00, d00);
        fma_raw<DT, VB>(acc, c.w01, d01);
        fma_raw<DT, VB>(acc, c.w10, d10);
        fma_raw<DT, VB>(acc, c.w11, d11);
    }
    store_raw<DT, VB>(a.out, (int64_t)n * a.img_out_elems + (int64_t)pix * a.C + g * a.Cg + lane_in_unit * NE, acc);
}

template <int DT, int VB, int SM>
void launch_k(const KArgs& a, int block, int64_t grid, hipStream_t stream)
{
    const uint32_t total = (uint32_t)grid;
    // renumbered per XCD (per_xcd > 0) when an image fits in one XCD's L2
    const uint32_t per_xcd = a.img_x_bytes <= kL2PerXcd ? (total + 7) / 8 : 0u;
    const uint32_t launched = per_xcd ? per_xcd * 8 : total;
    if (a.K == 3)
        hipLaunchKernelGGL((k_direct<DT, VB, 3, SM>), dim3(launched), dim3(block), 0, stream, a, total, per_xcd);
    else
        hipLaunchKernelGGL((k_direct<DT, VB, 0, SM>), dim3(launched), dim3(block), 0, stream, a, total, per_xcd);
}

template <int DT, int VB>
hipError_t launch_vb(const KArgs& a, int block, int64_t grid, hipStream_t stream)
{
    if (a.softmax) launch_k<DT, VB, 1>(a, block, grid, stream);
    else launch_k<DT, VB, 0>(a, block, grid, stream);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const KArgs& a, int block, int64_t grid, hipStream_t stream)
{
    switch (a.vec_bytes) {
        case 16: return launch_vb<DT, 16>(a, block, grid, stream);
        case 8: return launch_vb<DT, 8>(a, block, grid, stream);
        case 4: return launch_vb<DT, 4>(a, block, grid, stream);
        case 2: if constexpr (DT != DCNV4_F32) return launch_vb<DT, 2>(a, block, grid, stream); break;
        default: break;
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_direct(const KArgs& a, int dtype, int block, int64_t grid, hipStream_t stream)
{
    switch (dtype) {
        case DCNV4_F32: return launch_dt<DCNV4_F32>(a, block, grid, stream);
        case DCNV4_F16: return launch_dt<DCNV4_F16>(a, block, grid, stream);
        case DCNV4_BF16: return launch_dt<DCNV4_BF16>(a, block, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dcnv4

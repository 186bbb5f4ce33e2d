// DCNv4 module forward: the steps around the operator (include/dcnv4_module.h).
//
// The module: jsqmd.com/news/933833 ("不只是卷积的平替：我把DCNv4塞进Stable
// Diffusion的U-Net里"), section 2, the DCNv4Block example and item 2 of the
// list before it (a 1x1 channel projection, a normalisation, one predictor
// of offsets and weights: depthwise 3x3 then 1x1 to 3*G*P channels); centre-
// feature scaling through a sigmoid: pwwt.cn/news/2159231 section "进阶优化建议".
//
// Kernels (each step's result rounded once to the I/O type):
//   k_gemm       rows @ W^T + b on the matrix cores: one wave per 16 rows,
//                MFMA 16x16x16 (f16, bf16) or 16x16x4 (f32) with binary32
//                accumulation, 8 column blocks of 16 per pass so that a row
//                fragment is loaded once per pass.  The projections and the
//                predictor are dense contractions over the channels, the one
//                part of the module that is.
//   k_gn_partial / k_gn_finalize
//                group-norm statistics: binary64 sums per (image, slice of
//                pixels, channel), then per (image, group) in a fixed order
//                (reproducible), mean and 1/sqrt(var + eps).
//   k_norm       applies the group norm (or computes and applies a layer norm,
//                one wave per pixel, binary64 sums) -> xn.
//   k_dw3x3      depthwise 3x3, zero padding -> d.
//   k_gate       centre-feature gate y * (1 - s) + xn * s.
// The operator in between is the dcnv4_forward_ex kernel family on xn and the
// predictor's rows, read in place with the rows' stride.

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "dcnv4.h"
#include "dcnv4_device.h"
#include "dcnv4_internal.h"
#include "dcnv4_module.h"
#include "dcnv4_module_internal.h"

namespace dcnv4 {
namespace {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

template <int DT> struct Mfma;

// f16: A[i][k] for lane i + 16 * (k / 4), element k % 4 (4 consecutive k per
// lane, k step 16); B likewise by column; D rows 4 * (lane / 16) + r, column
// lane % 16.
template <> struct Mfma<DCNV4_F16> {
    static constexpr int kK = 16, kPer = 4;
    using Frag = h4;
    static __device__ __forceinline__ Frag load(__amdgpu_buffer_rsrc_t r, uint32_t off)
    {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
        return __builtin_bit_cast(Frag, v);
    }
    static __device__ __forceinline__ f4 mma(Frag a, Frag b, f4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mfma<DCNV4_BF16> {
    static constexpr int kK = 16, kPer = 4;
    using Frag = s4;
    static __device__ __forceinline__ Frag load(__amdgpu_buffer_rsrc_t r, uint32_t off)
    {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
        return __builtin_bit_cast(Frag, v);
    }
    static __device__ __forceinline__ f4 mma(Frag a, Frag b, f4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
};

// f32: one k per lane, A[i][k] for lane i + 16 * k, k step 4.
template <> struct Mfma<DCNV4_F32> {
    static constexpr int kK = 4, kPer = 1;
    using Frag = float;
    static __device__ __forceinline__ Frag load(__amdgpu_buffer_rsrc_t r, uint32_t off)
    {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
    }
    static __device__ __forceinline__ f4 mma(Frag a, Frag b, f4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// Column blocks of 16 per pass (accumulators held: 4 registers each), and
// the k chunk of the weight tile staged in LDS per step of the pass.
constexpr int kGemmBlocks = 8;
constexpr int kGemmCols = 16 * kGemmBlocks;
template <int DT> constexpr int kGemmKc = DT == DCNV4_F32 ? 32 : 64;
// LDS row pitch of the weight tile (elements): rows 4 (f32) or 8 (16-bit)
// bytes longer than the chunk, so that the 16 lanes reading one fragment
// column from 16 rows fall on different banks.
template <int DT> constexpr int kGemmPitch = kGemmKc<DT> + (DT == DCNV4_F32 ? 1 : 4);
constexpr int kGemmOutPitch = kGemmCols + 2;

// out[m][n] = round(sum_k a[m][k] * w[n][k] + bias[n]) for m < M, n < Nn.
// a: rows of lda elements (K used), w: [Nn][K] dense, out: rows of ldo.
// A workgroup of 4 waves takes 64 rows; per pass of 128 columns the weight
// tile goes through LDS in k chunks (each weight element read once per
// workgroup and pass), each wave reads its 16 rows' fragments from global
// memory (a chunk's loads issued together), and the results are gathered in
// LDS per wave and written row by row, consecutive lanes on consecutive
// columns.  K is a multiple of 4 for 16-bit types (8-byte loads).  Reads past
// a row's K-th element or past the last row or column return zero (buffer
// range checks), so ragged edges need no branches in the main loop.
template <int DT>
__global__ void __launch_bounds__(256) k_gemm(const void* __restrict__ a, int64_t lda, const void* __restrict__ w,
                                              const float* __restrict__ bias, void* __restrict__ out, int64_t ldo,
                                              int64_t M, int K, int Nn)
{
    using MF = Mfma<DT>;
    using E = Elem<DT>;
    using S = typename E::S;
    constexpr int s = E::kBytes;
    constexpr int KC = kGemmKc<DT>, WP = kGemmPitch<DT>;
    constexpr int STEPS = KC / MF::kK;
    __shared__ S wt[kGemmCols * WP];
    __shared__ S ot[4][16 * kGemmOutPitch];
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const int64_t row0 = (int64_t)blockIdx.x * 64 + wave * 16;
    const int rows_here = row0 < M ? (int)min<int64_t>(16, M - row0) : 0;
    const char* abase = static_cast<const char*>(a) + (rows_here ? row0 : 0) * lda * s;
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(abase, rows_here ? (uint32_t)(((int64_t)(rows_here - 1) * lda + K) * s) : 0u);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w, (uint32_t)((int64_t)Nn * K * s));
    const uint32_t li = lane & 15u, lk = lane >> 4;      // row (or column) and k group of this lane
    const int kq = MF::kPer * (int)lk;                     // first k of this lane in a step
    constexpr int EPL = DT == DCNV4_F32 ? 1 : 4;           // elements per staging load
    for (int n0 = 0; n0 < Nn; n0 += kGemmCols) {
        f4 acc[kGemmBlocks];
#pragma unroll
        for (int b = 0; b < kGemmBlocks; ++b) acc[b] = f4{0.f, 0.f, 0.f, 0.f};
        for (int kc0 = 0; kc0 < K; kc0 += KC) {
            // this wave's A fragments of the chunk, requested before the tile
            typename MF::Frag fa[STEPS];
#pragma unroll
            for (int st = 0; st < STEPS; ++st) {
                const int k = kc0 + st * MF::kK + kq;
                const bool ain = ((int)li < rows_here) & (k < K);
                fa[st] = MF::load(ra, ain ? (uint32_t)(((int64_t)li * lda + k) * s) : kOobOffset);
            }
            __syncthreads();   // the previous chunk's tile is consumed
            for (int e = threadIdx.x * EPL; e < kGemmCols * KC; e += 256 * EPL) {
                const int r = e / KC, c = e - r * KC;
                const int n = n0 + r, k = kc0 + c;
                const bool in = (n < Nn) & (k < K);
                const uint32_t off = in ? (uint32_t)(((int64_t)n * K + k) * s) : kOobOffset;
                if constexpr (EPL == 4) {
                    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rw, (int)off, 0, 0);
                    *reinterpret_cast<u32x2*>(&wt[r * WP + c]) = v;
                } else {
                    wt[r * WP + c] = __builtin_bit_cast(S, __builtin_amdgcn_raw_buffer_load_b32(rw, (int)off, 0, 0));
                }
            }
            __syncthreads();
#pragma unroll
            for (int st = 0; st < STEPS; ++st) {
#pragma unroll
                for (int b = 0; b < kGemmBlocks; ++b) {
                    if (n0 + 16 * b >= Nn) break;   // (uniform) no column of this block exists
                    const S* src = &wt[(16 * b + li) * WP + st * MF::kK + kq];
                    typename MF::Frag fb;
                    if constexpr (EPL == 4)
                        fb = __builtin_bit_cast(typename MF::Frag, *reinterpret_cast<const u32x2*>(src));
                    else
                        fb = *src;
                    acc[b] = MF::mma(fa[st], fb, acc[b]);
                }
            }
        }
        // bias, one rounding, through this wave's LDS tile to row-wise stores
        const int ncols = min(kGemmCols, Nn - n0);
#pragma unroll
        for (int b = 0; b < kGemmBlocks; ++b) {
            const int col = 16 * b + (int)li;
            if (col >= ncols) continue;
            const float bn = bias[n0 + col];
#pragma unroll
            for (int r = 0; r < 4; ++r) ot[wave][(4 * (int)lk + r) * kGemmOutPitch + col] = E::from_f(acc[b][r] + bn);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (int r = 0; r < rows_here; ++r) {
            S* orow = static_cast<S*>(out) + (row0 + r) * ldo + n0;
            for (int c = (int)lane; c < ncols; c += 64) orow[c] = ot[wave][r * kGemmOutPitch + c];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// Group-norm partial sums: block (n, slice) sums xp over its slice of the
// image's pixels per channel, in binary64, in a fixed order:
// part[((n * slices + slice) * C + c) * 2 + {0, 1}] = (sum v, sum v^2).
// Threads t < q * C (q = 256 / C, at least 1) take channel t % C and every
// q-th pixel from t / C; C > 256 loops the channels.
template <int DT>
__global__ void __launch_bounds__(256) k_gn_partial(const void* __restrict__ xp, double* __restrict__ part,
                                                    int HW, int C, int slices)
{
    using E = Elem<DT>;
    __shared__ double red[2][256];
    const int n = blockIdx.x / slices, slice = blockIdx.x % slices;
    const int p0 = (int)((int64_t)HW * slice / slices), p1 = (int)((int64_t)HW * (slice + 1) / slices);
    const typename E::S* x = static_cast<const typename E::S*>(xp) + (int64_t)n * HW * C;
    const int q = C < 256 ? 256 / C : 1;
    for (int cb = 0; cb < C; cb += 256) {
        const int t = threadIdx.x;
        const int c = cb + (C < 256 ? t % C : t);
        const int j = C < 256 ? t / C : 0;
        double s1 = 0.0, s2 = 0.0;
        if (c < C && j < q) {
            for (int p = p0 + j; p < p1; p += q) {
                const double v = (double)E::to_f(x[(int64_t)p * C + c]);
                s1 += v;
                s2 += v * v;
            }
        }
        red[0][t] = s1;
        red[1][t] = s2;
        __syncthreads();
        if (C < 256) {
            if (t < C) {
                double a1 = 0.0, a2 = 0.0;
                for (int jj = 0; jj < q; ++jj) {
                    a1 += red[0][jj * C + t];
                    a2 += red[1][jj * C + t];
                }
                double* o = part + (((int64_t)n * slices + slice) * C + t) * 2;
                o[0] = a1;
                o[1] = a2;
            }
        } else if (c < C) {
            double* o = part + (((int64_t)n * slices + slice) * C + c) * 2;
            o[0] = red[0][t];
            o[1] = red[1][t];
        }
        __syncthreads();
    }
}

// stat[(n * groups + g) * 2 + {0, 1}] = (mean, 1 / sqrt(var + eps)) from the
// partial sums, slices then channels in order.
__global__ void __launch_bounds__(256) k_gn_finalize(const double* __restrict__ part, float* __restrict__ stat,
                                                     int N, int HW, int C, int groups, int slices, float eps)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= N * groups) return;
    const int n = i / groups, g = i % groups, cpg = C / groups;
    double s1 = 0.0, s2 = 0.0;
    for (int sl = 0; sl < slices; ++sl)
        for (int c = g * cpg; c < (g + 1) * cpg; ++c) {
            const double* p = part + (((int64_t)n * slices + sl) * C + c) * 2;
            s1 += p[0];
            s2 += p[1];
        }
    const double cnt = (double)HW * cpg;
    const double mean = s1 / cnt;
    double var = s2 / cnt - mean * mean;
    var = var > 0.0 ? var : 0.0;
    stat[i * 2] = (float)mean;
    stat[i * 2 + 1] = (float)(1.0 / sqrt(var + (double)eps));
}

// VE consecutive elements of the I/O type as binary32 (VE = 1, or one
// 16-byte vector), and back with one rounding each.
template <int DT, int VE>
__device__ __forceinline__ void load_vals(const void* p, float* v)
{
    using E = Elem<DT>;
    if constexpr (VE == 1) {
        v[0] = E::to_f(*static_cast<const typename E::S*>(p));
    } else {
        static_assert(VE == kPerVec<DT>, "one 16-byte vector");
        const u32x4 q = *static_cast<const u32x4*>(p);
        const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (DT == DCNV4_F32) {
                v[i] = __uint_as_float(d[i]);
            } else {
                v[2 * i] = E::raw_to_f(d[i] & 0xffffu);
                v[2 * i + 1] = E::raw_to_f(d[i] >> 16);
            }
        }
    }
}

template <int DT, int VE>
__device__ __forceinline__ void store_vals(void* p, const float* v)
{
    using E = Elem<DT>;
    if constexpr (VE == 1) {
        *static_cast<typename E::S*>(p) = E::from_f(v[0]);
    } else {
        *static_cast<u32x4*>(p) = pack_vec16<DT>(v);
    }
}

// xn = round((xp - mean) * rstd * gamma + beta), VE channels per thread.
// Group norm: (mean, rstd) of each channel's group from `stat`, one thread
// per (pixel, VE channels).  Layer norm: the pixel's statistics computed
// here by a segment of lpp lanes (a power of two covering its C / VE chunks;
// 64 / lpp pixels per wave), binary64 sums, butterflies within the segment.
template <int DT, int LAYER, int VE>
__global__ void __launch_bounds__(256) k_norm(const void* __restrict__ xp, void* __restrict__ xn,
                                              const float* __restrict__ stat, const float* __restrict__ gamma,
                                              const float* __restrict__ beta, int64_t npix, int HW, int C,
                                              int groups, float eps, int lpp)
{
    using E = Elem<DT>;
    constexpr int s = E::kBytes;
    const int chunks = C / VE;
    if (!LAYER) {
        const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
        if (i >= npix * chunks) return;
        const int64_t pix = i / chunks;
        const int c0 = (int)(i - pix * chunks) * VE;
        const int n = (int)(pix / HW), cpg = C / groups;
        float v[VE];
        load_vals<DT, VE>(static_cast<const char*>(xp) + (pix * C + c0) * s, v);
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            const float* st = stat + ((int64_t)n * groups + (c0 + e) / cpg) * 2;
            v[e] = fmaf((v[e] - st[0]) * st[1], gamma[c0 + e], beta[c0 + e]);
        }
        store_vals<DT, VE>(static_cast<char*>(xn) + (pix * C + c0) * s, v);
        return;
    }
    const int lane = threadIdx.x & 63;
    const int sub = lane & (lpp - 1);
    const int64_t pix = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / lpp) + lane / lpp;
    const bool live = pix < npix;
    const char* x = static_cast<const char*>(xp) + (live ? pix : 0) * C * s;
    double s1 = 0.0, s2 = 0.0;
    if (live) {
        for (int j = sub; j < chunks; j += lpp) {
            float v[VE];
            load_vals<DT, VE>(x + (int64_t)j * VE * s, v);
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                s1 += (double)v[e];
                s2 += (double)v[e] * (double)v[e];
            }
        }
    }
    for (int off = lpp >> 1; off >= 1; off >>= 1) {
        s1 += __shfl_xor(s1, off);
        s2 += __shfl_xor(s2, off);
    }
    if (!live) return;
    const double m = s1 / C;
    double var = s2 / C - m * m;
    var = var > 0.0 ? var : 0.0;
    const float mean = (float)m, rstd = (float)(1.0 / sqrt(var + (double)eps));
    char* o = static_cast<char*>(xn) + pix * C * s;
    for (int j = sub; j < chunks; j += lpp) {
        float v[VE];
        load_vals<DT, VE>(x + (int64_t)j * VE * s, v);
#pragma unroll
        for (int e = 0; e < VE; ++e) v[e] = fmaf((v[e] - mean) * rstd, gamma[j * VE + e], beta[j * VE + e]);
        store_vals<DT, VE>(o + (int64_t)j * VE * s, v);
    }
}

// d = round(b[c] + sum_{i,j} w[c][i][j] * xn[h + i - 1][w + j - 1][c]), zero
// padding, taps in row-major order; one thread per (pixel, VE channels).
// LDSW: the taps and biases are first copied to LDS (C * 10 floats), so that
// each thread's 9 * VE tap reads are LDS reads rather than global loads.
template <int DT, int VE, int LDSW>
__global__ void __launch_bounds__(256) k_dw3x3(const void* __restrict__ xn, void* __restrict__ d,
                                               const float* __restrict__ w, const float* __restrict__ b,
                                               int N, int H, int W, int C)
{
    using E = Elem<DT>;
    constexpr int s = E::kBytes;
    extern __shared__ float wl[];
    const float* wt = w;
    const float* bt = b;
    if (LDSW) {
        for (int i = threadIdx.x; i < C * 9; i += blockDim.x) wl[i] = w[i];
        for (int i = threadIdx.x; i < C; i += blockDim.x) wl[C * 9 + i] = b[i];
        __syncthreads();
        wt = wl;
        bt = wl + C * 9;
    }
    const int chunks = C / VE;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)N * H * W * chunks) return;
    const int64_t pix = i / chunks;
    const int c0 = (int)(i - pix * chunks) * VE;
    const int wx = (int)(pix % W), hy = (int)((pix / W) % H);
    const int64_t img = pix / ((int64_t)H * W);
    const char* x = static_cast<const char*>(xn) + (img * H * W * C + c0) * s;
    float acc[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] = bt[c0 + e];
#pragma unroll
    for (int ii = 0; ii < 3; ++ii) {
        const int y = hy + ii - 1;
        if (y < 0 || y >= H) continue;
#pragma unroll
        for (int jj = 0; jj < 3; ++jj) {
            const int xx = wx + jj - 1;
            if (xx < 0 || xx >= W) continue;
            float v[VE];
            load_vals<DT, VE>(x + ((int64_t)y * W + xx) * C * s, v);
#pragma unroll
            for (int e = 0; e < VE; ++e) acc[e] = fmaf(wt[(c0 + e) * 9 + ii * 3 + jj], v[e], acc[e]);
        }
    }
    store_vals<DT, VE>(static_cast<char*>(d) + (pix * C + c0) * s, acc);
}

// gated = round(y * (1 - s) + xn * s), s = sigmoid(rows[pix][gate0 + c / Cg]);
// one thread per (pixel, VE channels).
template <int DT, int VE>
__global__ void __launch_bounds__(256) k_gate(const void* __restrict__ y, const void* __restrict__ xn,
                                              const void* __restrict__ rows, int64_t rstride, int gate0,
                                              void* __restrict__ out, int64_t npix, int C, int Cg)
{
    using E = Elem<DT>;
    constexpr int s = E::kBytes;
    const int chunks = C / VE;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= npix * chunks) return;
    const int64_t pix = i / chunks;
    const int c0 = (int)(i - pix * chunks) * VE;
    const int64_t at = (pix * C + c0) * s;
    float yv[VE], xv[VE];
    load_vals<DT, VE>(static_cast<const char*>(y) + at, yv);
    load_vals<DT, VE>(static_cast<const char*>(xn) + at, xv);
    const typename E::S* lg = static_cast<const typename E::S*>(rows) + pix * rstride + gate0;
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        const float t = E::to_f(lg[(c0 + e) / Cg]);
        const float sg = 1.0f / (1.0f + expf(-t));
        yv[e] = yv[e] * (1.0f - sg) + xv[e] * sg;
    }
    store_vals<DT, VE>(static_cast<char*>(out) + at, yv);
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <int DT>
hipError_t run(const ModuleProblem& m, hipStream_t st)
{
    const int64_t npix = (int64_t)m.N * m.H * m.W;
    const int C = m.G * m.Cg, HW = m.H * m.W;
    char* ws = static_cast<char*>(m.workspace);
    const ModuleLayout& L = m.layout;
    void* xp = ws + L.xp;
    void* xn = L.xn >= 0 ? ws + L.xn : xp;
    void* d = ws + L.d;
    void* rows = ws + L.rows;
    const int64_t gblocks = cdiv(npix, 64);
    // elementwise steps: one 16-byte vector per thread when the channels
    // split into whole vectors (the workspace regions are 256-byte aligned)
    constexpr int VE = kPerVec<DT>;
    const bool vec = C % VE == 0 && (uintptr_t)m.out % 16 == 0;
    // 1. projection
    hipLaunchKernelGGL(k_gemm<DT>, dim3((unsigned)gblocks), dim3(256), 0, st, m.x_in, (int64_t)m.Cin, m.w.w_in,
                       m.w.b_in, xp, (int64_t)C, npix, m.Cin, C);
    // 2. normalisation
    if (m.norm == DCNV4_NORM_GROUP) {
        double* part = reinterpret_cast<double*>(ws + L.stats);
        float* stat = reinterpret_cast<float*>(ws + L.stats + L.stat_offset);
        hipLaunchKernelGGL(k_gn_partial<DT>, dim3((unsigned)(m.N * L.slices)), dim3(256), 0, st, xp, part, HW, C,
                           L.slices);
        hipLaunchKernelGGL(k_gn_finalize, dim3((unsigned)cdiv((int64_t)m.N * m.norm_groups, 256)), dim3(256), 0, st,
                           part, stat, m.N, HW, C, m.norm_groups, L.slices, m.eps);
        if (vec)
            hipLaunchKernelGGL((k_norm<DT, 0, VE>), dim3((unsigned)cdiv(npix * (C / VE), 256)), dim3(256), 0, st, xp,
                               xn, stat, m.w.gamma, m.w.beta, npix, HW, C, m.norm_groups, m.eps, 1);
        else
            hipLaunchKernelGGL((k_norm<DT, 0, 1>), dim3((unsigned)cdiv(npix * C, 256)), dim3(256), 0, st, xp, xn,
                               stat, m.w.gamma, m.w.beta, npix, HW, C, m.norm_groups, m.eps, 1);
    } else if (m.norm == DCNV4_NORM_LAYER) {
        // a segment of lpp lanes (a power of two, at most 64) per pixel
        const int chunks = vec ? C / VE : C;
        int lpp = 1;
        while (lpp < chunks && lpp < 64) lpp <<= 1;
        const unsigned grid = (unsigned)cdiv(npix, 4 * (64 / lpp));
        if (vec)
            hipLaunchKernelGGL((k_norm<DT, 1, VE>), dim3(grid), dim3(256), 0, st, xp, xn, nullptr, m.w.gamma,
                               m.w.beta, npix, HW, C, 1, m.eps, lpp);
        else
            hipLaunchKernelGGL((k_norm<DT, 1, 1>), dim3(grid), dim3(256), 0, st, xp, xn, nullptr, m.w.gamma,
                               m.w.beta, npix, HW, C, 1, m.eps, lpp);
    }
    // 3. depthwise 3x3, 4. predictor
    {
        // taps through LDS when they fit in 64 KiB (up to 1638 channels)
        const size_t wbytes = (size_t)C * 10 * sizeof(float);
        const bool lw = wbytes <= 64 * 1024;
        const unsigned grid = (unsigned)cdiv(npix * (vec ? C / VE : C), 256);
        if (vec && lw)
            hipLaunchKernelGGL((k_dw3x3<DT, VE, 1>), dim3(grid), dim3(256), wbytes, st, xn, d, m.w.w_dw, m.w.b_dw,
                               m.N, m.H, m.W, C);
        else if (vec)
            hipLaunchKernelGGL((k_dw3x3<DT, VE, 0>), dim3(grid), dim3(256), 0, st, xn, d, m.w.w_dw, m.w.b_dw, m.N,
                               m.H, m.W, C);
        else if (lw)
            hipLaunchKernelGGL((k_dw3x3<DT, 1, 1>), dim3(grid), dim3(256), wbytes, st, xn, d, m.w.w_dw, m.w.b_dw,
                               m.N, m.H, m.W, C);
        else
            hipLaunchKernelGGL((k_dw3x3<DT, 1, 0>), dim3(grid), dim3(256), 0, st, xn, d, m.w.w_dw, m.w.b_dw, m.N,
                               m.H, m.W, C);
    }
    hipLaunchKernelGGL(k_gemm<DT>, dim3((unsigned)gblocks), dim3(256), 0, st, d, (int64_t)C, m.w.w_pred,
                       m.w.b_pred, rows, L.rows_stride, npix, C, L.R);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // 5. the operator on xn with the predictor's rows read in place
    void* y = L.y >= 0 ? ws + L.y : m.out;
    {
        const int s = DT == DCNV4_F32 ? 4 : 2;
        Problem p;
        memset(&p, 0, sizeof p);
        p.x = xn;
        p.off = rows;
        p.msk = static_cast<const char*>(rows) + (int64_t)2 * m.G * L.P * s;
        p.out = y;
        p.N = m.N; p.H = m.H; p.W = m.W; p.G = m.G; p.Cg = m.Cg; p.K = 3; p.P = L.P;
        p.stride = 1; p.pad = 1; p.dil = 1; p.Ho = m.H; p.Wo = m.W;
        p.remove_center = m.remove_center;
        p.softmax = 0;
        p.off_row = L.rows_stride;
        p.mask_row = L.rows_stride;
        p.offset_scale = m.offset_scale;
        p.dtype = DT;
        p.cus = m.cus;
        Plan plan;
        make_plan(p, &plan);
        e = launch_forward(p, plan, st);
        if (e != hipSuccess) return e;
    }
    // 6. centre-feature gate, 7. output projection
    void* last = y;
    if (m.center_scale) {
        void* g = L.gated >= 0 ? ws + L.gated : m.out;
        if (vec)
            hipLaunchKernelGGL((k_gate<DT, VE>), dim3((unsigned)cdiv(npix * (C / VE), 256)), dim3(256), 0, st, y, xn,
                               rows, L.rows_stride, 3 * m.G * L.P, g, npix, C, m.Cg);
        else
            hipLaunchKernelGGL((k_gate<DT, 1>), dim3((unsigned)cdiv(npix * C, 256)), dim3(256), 0, st, y, xn, rows,
                               L.rows_stride, 3 * m.G * L.P, g, npix, C, m.Cg);
        last = g;
    }
    if (m.out_proj)
        hipLaunchKernelGGL(k_gemm<DT>, dim3((unsigned)gblocks), dim3(256), 0, st, last, (int64_t)C, m.w.w_out,
                           m.w.b_out, m.out, (int64_t)m.Cout, npix, C, m.Cout);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_module(const ModuleProblem& m, hipStream_t stream)
{
    switch (m.dtype) {
        case DCNV4_F32: return run<DCNV4_F32>(m, stream);
        case DCNV4_F16: return run<DCNV4_F16>(m, stream);
        case DCNV4_BF16: return run<DCNV4_BF16>(m, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dcnv4

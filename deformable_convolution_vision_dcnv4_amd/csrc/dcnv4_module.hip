// DCNv4 module forward: the steps around the operator (include/dcnv4_module.h).
//
// The module: jsqmd.com/news/933833 ("不只是卷积的平替：我把DCNv4塞进Stable
// Diffusion的U-Net里"), section 2, the DCNv4Block example and item 2 of the
// list before it (a 1x1 channel projection, a normalisation, one predictor
// of offsets and weights: depthwise 3x3 then 1x1 to 3*G*P channels); centre-
// feature scaling through a sigmoid: pwwt.cn/news/2159231 section "进阶优化建议".
//
// Kernels (each step's result rounded once to the I/O type):
//   k_gemmv      rows @ W^T + b on the matrix cores (MFMA 16x16x16 f16/bf16,
//                16x16x4 f32, binary32 accumulation) for 16-byte aligned rows
//                of at most 640 bytes: the weights held in LDS across a
//                grid-stride walk over row tiles; optionally applies the
//                centre-feature gate to its rows as they are read.  k_gemm:
//                the general form.  The projections and the predictor are
//                dense contractions over the channels, the one part of the
//                module that is.
//   k_gn_partial / k_gn_finalize
//                group-norm statistics: binary64 sums per (image, slice of
//                pixels, channel), then per (image, group) in a fixed order
//                (reproducible), mean and 1/sqrt(var + eps).
//   k_norm       applies the group norm (or computes and applies a layer norm,
//                one wave per pixel, binary64 sums) -> xn.
//   k_dw3x3v     depthwise 3x3, zero padding -> d, runs of four pixels per
//                thread with the taps in LDS; k_dw3x3: the general form.
//   k_gate       centre-feature gate y * (1 - s) + xn * s, when the output
//                projection does not apply it.
// The operator in between is the dcnv4_forward_ex kernel family on xn and the
// predictor's rows, read in place with the rows' stride.

#include <math.h>

#include <algorithm>
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
    // step e's fragment (elements 4e .. 4e + 3) of a 16-byte vector
    static __device__ __forceinline__ Frag part(u32x4 v, int e)
    {
        const u32x2 d = e == 0 ? u32x2{v.x, v.y} : u32x2{v.z, v.w};
        return __builtin_bit_cast(Frag, d);
    }
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
    static __device__ __forceinline__ Frag part(u32x4 v, int e)
    {
        const u32x2 d = e == 0 ? u32x2{v.x, v.y} : u32x2{v.z, v.w};
        return __builtin_bit_cast(Frag, d);
    }
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
    static __device__ __forceinline__ Frag part(u32x4 v, int e)
    {
        return __uint_as_float(e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w);
    }
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

// Thread index -> (pixel, channel chunk) for the elementwise kernels, with
// unsigned 32-bit divisions when the grid's threads number below 2^31 (the
// common case; 64-bit division is a long instruction sequence).
__device__ __forceinline__ bool narrow_grid()
{
    return (uint64_t)gridDim.x * blockDim.x <= 0x7fffffffull;
}

__device__ __forceinline__ void split_index(int64_t i, int chunks, bool narrow, int64_t& pix, int& chunk)
{
    if (narrow) {
        const uint32_t ii = (uint32_t)i, p = ii / (uint32_t)chunks;
        pix = p;
        chunk = (int)(ii - p * (uint32_t)chunks);
    } else {
        pix = i / chunks;
        chunk = (int)(i - pix * chunks);
    }
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

// Vector form of k_gemm for 16-byte aligned operands with K * s a multiple
// of 16 and at most KV * 64 bytes.  A workgroup of 8 waves loads the weights
// of its column range [n0, n0 + NB) for all of K into LDS once (zero past K
// and past the last column) and then walks row tiles of 128 rows (16 per
// wave) with a grid stride, requesting the next tile's rows before the
// current tile's products.  Lane (i, kg) = (lane % 16, lane / 16) reads row
// i's elements [(4v + kg) E, (4v + kg + 1) E) as its 16-byte vector v
// (E = 16 / s) and feeds them to E / kPer MFMA steps, kPer at a time; the
// weight fragment of the same lane and step is the same k range of column j
// from LDS.  Every step thus pairs each k with itself: a permutation of the
// contraction's products over the steps, accumulated in binary32.  The
// results go through a per-wave LDS tile to 16-byte row-wise stores.
// Grid: passes * GR workgroups, workgroup b taking pass b % passes.
constexpr int kGemmvWaves = 8;
constexpr int kGemmvMaxBlocks = 10;   // column blocks of 16 per pass (NB <= 160)

// The centre-feature gate applied while the output projection reads its
// rows (GATE): the projection's input row is gated = round(y * (1 - s) +
// xn * s), s = sigmoid(rows[pix][gate0 + c / Cg]), the same operations as
// k_gate, so the same values; y is the kernel's `a`, xn has the same layout.
struct GateSrc {
    const void* xn;
    const void* rows;
    int64_t rstride;   // elements per pixel of rows
    int gate0, Cg;
};

// One wave's 16 rows of tile t (128 rows per tile) as KV 16-byte vectors per
// lane, vector v of lane (li, kg) holding row li's bytes [(4v + kg) 16, + 16);
// zeros past M, past K and for t >= T.  GATE: also xn's vectors and the raw
// gate logit of each vector's group (a vector lies in one group).
template <int DT, int KV, int GATE>
__device__ __forceinline__ void gemmv_rows(const void* a, int64_t lda, int64_t M, int K, int64_t t, int64_t T,
                                           uint32_t wave, int li, int kg, const GateSrc& gs, u32x4 (&fa)[KV],
                                           u32x4 (&fx)[KV], uint32_t (&fl)[KV])
{
    constexpr int s = Elem<DT>::kBytes;
    const int64_t r0 = t * 128 + wave * 16;
    const int rows_here = (t < T && r0 < M) ? (int)min<int64_t>(16, M - r0) : 0;
    const uint32_t span = rows_here ? (uint32_t)(((int64_t)(rows_here - 1) * lda + K) * s) : 0u;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(static_cast<const char*>(a) + (rows_here ? r0 : 0) * lda * s, span);
    const int kbytes = K * s;
#pragma unroll
    for (int v = 0; v < KV; ++v) {
        const int kb = (4 * v + kg) * 16;
        const bool in = (li < rows_here) & (kb < kbytes);
        fa[v] = buf_load16(ra, in ? (uint32_t)((int64_t)li * lda * s + kb) : kOobOffset);
    }
    if constexpr (GATE) {
        const __amdgpu_buffer_rsrc_t rx =
            make_rsrc(static_cast<const char*>(gs.xn) + (rows_here ? r0 : 0) * lda * s, span);
        const __amdgpu_buffer_rsrc_t rr = make_rsrc(
            static_cast<const char*>(gs.rows) + (rows_here ? r0 : 0) * gs.rstride * s,
            rows_here ? (uint32_t)((int64_t)rows_here * gs.rstride * s) : 0u);
#pragma unroll
        for (int v = 0; v < KV; ++v) {
            const int kb = (4 * v + kg) * 16;
            const bool in = (li < rows_here) & (kb < kbytes);
            fx[v] = buf_load16(rx, in ? (uint32_t)((int64_t)li * lda * s + kb) : kOobOffset);
            const int g = kb / s / gs.Cg;
            const uint32_t lo = in ? (uint32_t)(((int64_t)li * gs.rstride + gs.gate0 + g) * s) : kOobOffset;
            if constexpr (s == 4)
                fl[v] = __builtin_amdgcn_raw_buffer_load_b32(rr, (int)lo, 0, 0);
            else
                fl[v] = __builtin_amdgcn_raw_buffer_load_b16(rr, (int)lo, 0, 0);
        }
    }
}

// y's vector gated with xn's, one rounding per element (as k_gate).
template <int DT>
__device__ __forceinline__ u32x4 gate_vector(u32x4 y, u32x4 x, uint32_t logit_raw)
{
    constexpr int EV = kPerVec<DT>;
    const float tl = Elem<DT>::raw_to_f(logit_raw);
    const float sg = 1.0f / (1.0f + expf(-tl));
    float yv[EV], xv[EV];
    load_vals<DT, EV>(&y, yv);
    load_vals<DT, EV>(&x, xv);
#pragma unroll
    for (int e = 0; e < EV; ++e) yv[e] = yv[e] * (1.0f - sg) + xv[e] * sg;
    return pack_vec16<DT>(yv);
}

template <int DT, int KV, int GATE>
__global__ void __launch_bounds__(512) k_gemmv(const void* __restrict__ a, int64_t lda, const void* __restrict__ w,
                                               const float* __restrict__ bias, void* __restrict__ out, int64_t ldo,
                                               int64_t M, int K, int Nn, int NB, int passes, int wpitch, GateSrc gs)
{
    using MF = Mfma<DT>;
    using E = Elem<DT>;
    using S = typename E::S;
    constexpr int s = E::kBytes, EV = 16 / s, STEPS = EV / MF::kPer;
    extern __shared__ __align__(16) unsigned char lds[];
    const int pass = blockIdx.x % passes, GR = gridDim.x / passes, rg0 = blockIdx.x / passes;
    const int n0 = pass * NB, nbb = NB / 16;
    const int opitch = NB * s + 16;                        // bytes per row of the output tile
    unsigned char* wt = lds;                               // [NB][wpitch bytes]
    unsigned char* ot = lds + NB * wpitch + (threadIdx.x >> 6) * 16 * opitch;
    // weights: column n0 + r, bytes [0, KV * 64) of its k range, zero past K and Nn
    const int kbytes = K * s, vrow = KV * 4;                // 16-byte vectors per staged column
    for (int e = threadIdx.x; e < NB * vrow; e += blockDim.x) {
        const int r = e / vrow, c = e - r * vrow;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (n0 + r < Nn && c * 16 < kbytes)
            v = *reinterpret_cast<const u32x4*>(static_cast<const char*>(w) + (int64_t)(n0 + r) * kbytes + c * 16);
        *reinterpret_cast<u32x4*>(wt + r * wpitch + c * 16) = v;
    }
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const int li = (int)(lane & 15u), kg = (int)(lane >> 4);
    float bn[kGemmvMaxBlocks];
#pragma unroll
    for (int b = 0; b < kGemmvMaxBlocks; ++b) {
        const int col = n0 + 16 * b + li;
        bn[b] = (b < nbb && col < Nn) ? bias[col] : 0.f;
    }
    __syncthreads();
    const int64_t T = (M + 127) / 128;
    u32x4 fa[KV], fn[KV], xa[KV], xn_[KV];
    uint32_t la[KV], ln[KV];
    int64_t t = rg0;
    gemmv_rows<DT, KV, GATE>(a, lda, M, K, t, T, wave, li, kg, gs, fa, xa, la);
    for (; t < T; t += GR) {
        gemmv_rows<DT, KV, GATE>(a, lda, M, K, t + GR, T, wave, li, kg, gs, fn, xn_, ln);
        if constexpr (GATE) {
#pragma unroll
            for (int v = 0; v < KV; ++v) fa[v] = gate_vector<DT>(fa[v], xa[v], la[v]);
        }
        f4 acc[kGemmvMaxBlocks];
#pragma unroll
        for (int b = 0; b < kGemmvMaxBlocks; ++b) acc[b] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < KV; ++v) {
#pragma unroll
            for (int b = 0; b < kGemmvMaxBlocks; ++b) {
                if (b >= nbb) continue;   // (uniform)
                const u32x4 wv = *reinterpret_cast<const u32x4*>(wt + (16 * b + li) * wpitch + (4 * v + kg) * 16);
#pragma unroll
                for (int e = 0; e < STEPS; ++e) acc[b] = MF::mma(MF::part(fa[v], e), MF::part(wv, e), acc[b]);
            }
        }
        // bias, one rounding, to the wave's tile: row 4 * kg + r, column 16 * b + li
#pragma unroll
        for (int b = 0; b < kGemmvMaxBlocks; ++b) {
            if (b >= nbb) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *reinterpret_cast<S*>(ot + (4 * kg + r) * opitch + (16 * b + li) * s) = E::from_f(acc[b][r] + bn[b]);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int64_t r0 = t * 128 + wave * 16;
        const int cpr = NB / EV;                            // 16-byte chunks per tile row
        for (int c = (int)lane; c < 16 * cpr; c += 64) {
            const int r = c / cpr, q = c - r * cpr;
            const int col = n0 + q * EV;
            if (r0 + r >= M || col >= Nn) continue;
            const unsigned char* src = ot + r * opitch + q * 16;
            char* dst = static_cast<char*>(out) + ((r0 + r) * ldo + col) * s;
            if (col + EV <= Nn) {
                *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
            } else {
                for (int e = 0; e < Nn - col; ++e)
                    reinterpret_cast<S*>(dst)[e] = reinterpret_cast<const S*>(src)[e];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int v = 0; v < KV; ++v) {
            fa[v] = fn[v];
            if constexpr (GATE) {
                xa[v] = xn_[v];
                la[v] = ln[v];
            }
        }
    }
}

// Group-norm partial sums: block (n, slice) sums xp over its slice of the
// image's pixels per channel, in binary64, in a fixed order:
// part[((n * slices + slice) * C + c) * 2 + {0, 1}] = (sum v, sum v^2).
// Thread t takes the chunk of VE consecutive channels t % nb (one 16-byte
// vector when VE > 1; nb = the chunks of this pass, at most 256) and every
// q-th pixel of the slice from t / nb (q = 256 / nb), four pixels' loads in
// flight; the q row sums of each channel are then added in row order.
template <int DT, int VE>
__global__ void __launch_bounds__(256) k_gn_partial(const void* __restrict__ xp, double* __restrict__ part,
                                                    int HW, int C, int slices)
{
    using E = Elem<DT>;
    constexpr int s = E::kBytes;
    __shared__ double red[2][256 * VE];
    const int n = blockIdx.x / slices, slice = blockIdx.x % slices;
    const int p0 = (int)((int64_t)HW * slice / slices), p1 = (int)((int64_t)HW * (slice + 1) / slices);
    const char* x = static_cast<const char*>(xp) + (int64_t)n * HW * C * s;
    const int chunks = C / VE, t = threadIdx.x;
    for (int cb = 0; cb < chunks; cb += 256) {
        const int nb = min(256, chunks - cb), q = 256 / nb;
        const int j = t / nb, cv = cb + t % nb;
        double s1[VE], s2[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) s1[e] = s2[e] = 0.0;
        if (j < q) {
            const char* xc = x + (int64_t)cv * VE * s;
            int p = p0 + j;
            for (; p + 3 * q < p1; p += 4 * q) {
                float v[4][VE];
#pragma unroll
                for (int u = 0; u < 4; ++u) load_vals<DT, VE>(xc + (int64_t)(p + u * q) * C * s, v[u]);
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int e = 0; e < VE; ++e) {
                        const double d = (double)v[u][e];
                        s1[e] += d;
                        s2[e] += d * d;
                    }
            }
            for (; p < p1; p += q) {
                float v[VE];
                load_vals<DT, VE>(xc + (int64_t)p * C * s, v);
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    const double d = (double)v[e];
                    s1[e] += d;
                    s2[e] += d * d;
                }
            }
        }
        // entry (row j, channel ci of this pass) at j * nb * VE + ci
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            red[0][t * VE + e] = s1[e];
            red[1][t * VE + e] = s2[e];
        }
        __syncthreads();
        for (int ci = t; ci < nb * VE; ci += 256) {
            double a1 = 0.0, a2 = 0.0;
            for (int jj = 0; jj < q; ++jj) {
                a1 += red[0][jj * nb * VE + ci];
                a2 += red[1][jj * nb * VE + ci];
            }
            double* o = part + (((int64_t)n * slices + slice) * C + cb * VE + ci) * 2;
            o[0] = a1;
            o[1] = a2;
        }
        __syncthreads();
    }
}

// stat[(n * groups + g) * 2 + {0, 1}] = (mean, 1 / sqrt(var + eps)) from the
// partial sums: one wave per (image, group).  Lane l adds the group's
// (slice, channel) entries l, l + 64, ... in order; the 64 lane sums are then
// combined by a butterfly (the same tree on every run: reproducible).
__global__ void __launch_bounds__(256) k_gn_finalize(const double* __restrict__ part, float* __restrict__ stat,
                                                     int N, int HW, int C, int groups, int slices, float eps)
{
    const int lane = threadIdx.x & 63;
    const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= N * groups) return;   // whole waves
    const int n = i / groups, g = i % groups, cpg = C / groups;
    const int terms = slices * cpg;
    double s1 = 0.0, s2 = 0.0;
    for (int tt = lane; tt < terms; tt += 64) {
        const int sl = tt / cpg, c = g * cpg + (tt - sl * cpg);
        const double* p = part + (((int64_t)n * slices + sl) * C + c) * 2;
        s1 += p[0];
        s2 += p[1];
    }
    for (int off = 32; off >= 1; off >>= 1) {
        s1 += __shfl_xor(s1, off);
        s2 += __shfl_xor(s2, off);
    }
    if (lane != 0) return;
    const double cnt = (double)HW * cpg;
    const double mean = s1 / cnt;
    double var = s2 / cnt - mean * mean;
    var = var > 0.0 ? var : 0.0;
    stat[i * 2] = (float)mean;
    stat[i * 2 + 1] = (float)(1.0 / sqrt(var + (double)eps));
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
        const bool narrow = narrow_grid();
        int64_t pix;
        int ch;
        split_index(i, chunks, narrow, pix, ch);
        const int c0 = ch * VE;
        const int n = narrow ? (int)((uint32_t)pix / (uint32_t)HW) : (int)(pix / HW), cpg = C / groups;
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
// padding, taps in row-major order; one thread per (pixel, VE channels).  In
// the vector form a tap outside the image adds w * 0 (as zero padding does).
// LDSW: the taps are first copied to LDS transposed, tap-major ([9][C], then
// the C biases), so that a thread reads its VE channels of a tap as
// consecutive words and neighbouring threads neighbouring words.
template <int DT, int VE, int LDSW>
__global__ void __launch_bounds__(256) k_dw3x3(const void* __restrict__ xn, void* __restrict__ d,
                                               const float* __restrict__ w, const float* __restrict__ b,
                                               int N, int H, int W, int C)
{
    using E = Elem<DT>;
    constexpr int s = E::kBytes;
    extern __shared__ __align__(16) float wl[];
    if (LDSW) {
        for (int i = threadIdx.x; i < C * 9; i += blockDim.x) {
            const int c = i / 9, k = i - c * 9;
            wl[k * C + c] = w[i];
        }
        for (int i = threadIdx.x; i < C; i += blockDim.x) wl[C * 9 + i] = b[i];
        __syncthreads();
    }
    const int chunks = C / VE;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)N * H * W * chunks) return;
    const bool narrow = narrow_grid();
    int64_t pix, img;
    int ch, wx, hy;
    split_index(i, chunks, narrow, pix, ch);
    if (narrow) {
        const uint32_t p = (uint32_t)pix, q = p / (uint32_t)W;
        wx = (int)(p - q * (uint32_t)W);
        img = q / (uint32_t)H;
        hy = (int)(q - (uint32_t)img * (uint32_t)H);
    } else {
        wx = (int)(pix % W);
        hy = (int)((pix / W) % H);
        img = pix / ((int64_t)H * W);
    }
    const int c0 = ch * VE;
    // tap k of channel c: wl[k * C + c] (LDS) or w[c * 9 + k]
    auto tap = [&](int c, int k) { return LDSW ? wl[k * C + c] : w[c * 9 + k]; };
    float acc[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] = LDSW ? wl[C * 9 + c0 + e] : b[c0 + e];
    if constexpr (VE > 1) {
        // the nine neighbours' vectors requested together; a neighbour outside
        // the image reads zeros (buffer range check), so there is no branch
        const __amdgpu_buffer_rsrc_t r =
            make_rsrc(static_cast<const char*>(xn) + img * H * W * C * s, (uint32_t)((int64_t)H * W * C * s));
        u32x4 v[9];
#pragma unroll
        for (int k = 0; k < 9; ++k) {
            const int y = hy + k / 3 - 1, xx = wx + k % 3 - 1;
            const bool in = (y >= 0) & (y < H) & (xx >= 0) & (xx < W);
            v[k] = buf_load16(r, in ? (uint32_t)((((int64_t)y * W + xx) * C + c0) * s) : kOobOffset);
        }
#pragma unroll
        for (int k = 0; k < 9; ++k) {
            float f[VE], tk[VE];
            load_vals<DT, VE>(&v[k], f);
            if (LDSW) {
                // the VE taps as 16-byte LDS reads (c0 is a multiple of VE)
#pragma unroll
                for (int q = 0; q < VE / 4; ++q) {
                    const f4 t4 = *reinterpret_cast<const f4*>(&wl[k * C + c0 + 4 * q]);
                    tk[4 * q] = t4[0];
                    tk[4 * q + 1] = t4[1];
                    tk[4 * q + 2] = t4[2];
                    tk[4 * q + 3] = t4[3];
                }
            } else {
#pragma unroll
                for (int e = 0; e < VE; ++e) tk[e] = tap(c0 + e, k);
            }
#pragma unroll
            for (int e = 0; e < VE; ++e) acc[e] = fmaf(tk[e], f[e], acc[e]);
        }
    } else {
        const char* x = static_cast<const char*>(xn) + (img * H * W * C + c0) * s;
#pragma unroll
        for (int ii = 0; ii < 3; ++ii) {
            const int y = hy + ii - 1;
            if (y < 0 || y >= H) continue;
#pragma unroll
            for (int jj = 0; jj < 3; ++jj) {
                const int xx = wx + jj - 1;
                if (xx < 0 || xx >= W) continue;
                float f[VE];
                load_vals<DT, VE>(x + ((int64_t)y * W + xx) * C * s, f);
#pragma unroll
                for (int e = 0; e < VE; ++e) acc[e] = fmaf(tap(c0 + e, ii * 3 + jj), f[e], acc[e]);
            }
        }
    }
    store_vals<DT, VE>(static_cast<char*>(d) + (pix * C + c0) * s, acc);
}

// The depthwise 3x3 for 16-byte channel chunks with the taps in LDS: one
// thread per (row, run of PX pixels, chunk of VE channels).  Its (PX + 2) x 3
// neighbour vectors are requested together (zeros outside the image: buffer
// range check), each tap's VE values are read once from LDS (16-byte reads,
// tap-major layout) and applied to the PX outputs.  Per output the sum is
// the same as in k_dw3x3: bias, then the nine taps in row-major order.
template <int DT, int PX>
__global__ void __launch_bounds__(256) k_dw3x3v(const void* __restrict__ xn, void* __restrict__ d,
                                                const float* __restrict__ w, const float* __restrict__ b,
                                                int N, int H, int W, int C)
{
    using E = Elem<DT>;
    constexpr int s = E::kBytes, VE = kPerVec<DT>;
    extern __shared__ __align__(16) float wl[];
    for (int i = threadIdx.x; i < C * 9; i += blockDim.x) {
        const int c = i / 9, k = i - c * 9;
        wl[k * C + c] = w[i];
    }
    for (int i = threadIdx.x; i < C; i += blockDim.x) wl[C * 9 + i] = b[i];
    __syncthreads();
    const int chunks = C / VE, runs = (W + PX - 1) / PX;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)N * H * runs * chunks) return;
    const bool narrow = narrow_grid();
    int64_t t, img;
    int ch, run, hy;
    split_index(i, chunks, narrow, t, ch);
    if (narrow) {
        const uint32_t tt = (uint32_t)t, row = tt / (uint32_t)runs;
        run = (int)(tt - row * (uint32_t)runs);
        img = row / (uint32_t)H;
        hy = (int)(row - (uint32_t)img * (uint32_t)H);
    } else {
        const int64_t row = t / runs;
        run = (int)(t - row * runs);
        img = row / H;
        hy = (int)(row - img * H);
    }
    const int c0 = ch * VE, wx0 = run * PX;
    // one resource over the whole tensor (the host launches this kernel only
    // when it is under 2 GiB, so 32-bit offsets fit and stay below the
    // out-of-range offset): the same for every lane, where one per image
    // would make the compiler loop over the lanes' distinct resources at
    // every load
    const __amdgpu_buffer_rsrc_t r = make_rsrc(xn, (uint32_t)((int64_t)N * H * W * C * s));
    const uint32_t pstep = (uint32_t)C * s;                  // bytes per pixel
    float acc[PX][VE];
#pragma unroll
    for (int q = 0; q < VE / 4; ++q) {
        const f4 b4 = *reinterpret_cast<const f4*>(&wl[C * 9 + c0 + 4 * q]);
#pragma unroll
        for (int px = 0; px < PX; ++px)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[px][4 * q + e] = b4[e];
    }
    // one input row at a time: its PX + 2 vectors, then its three taps on the
    // PX outputs.  (With all three rows loaded up front the compiler widened
    // all 18 vectors at once, about 190 registers and two waves per SIMD.)
#pragma unroll
    for (int ii = 0; ii < 3; ++ii) {
        const int y = hy + ii - 1;
        const uint32_t o0 = (((uint32_t)img * (uint32_t)H + (uint32_t)y) * (uint32_t)W + (uint32_t)(wx0 - 1)) * pstep +
                            (uint32_t)c0 * s;
        u32x4 v[PX + 2];
#pragma unroll
        for (int j = 0; j < PX + 2; ++j) {
            const int xx = wx0 + j - 1;
            const bool in = (y >= 0) & (y < H) & (xx >= 0) & (xx < W);
            v[j] = buf_load16(r, in ? o0 + (uint32_t)j * pstep : kOobOffset);
        }
#pragma unroll
        for (int jj = 0; jj < 3; ++jj) {
            const int k = ii * 3 + jj;
            float tk[VE];
#pragma unroll
            for (int q = 0; q < VE / 4; ++q) {
                const f4 t4 = *reinterpret_cast<const f4*>(&wl[k * C + c0 + 4 * q]);
#pragma unroll
                for (int e = 0; e < 4; ++e) tk[4 * q + e] = t4[e];
            }
#pragma unroll
            for (int px = 0; px < PX; ++px) {
                float f[VE];
                load_vals<DT, VE>(&v[px + jj], f);
#pragma unroll
                for (int e = 0; e < VE; ++e) acc[px][e] = fmaf(tk[e], f[e], acc[px][e]);
            }
        }
        // the next row's loads are issued after this row's multiply-adds (the
        // accumulators are pinned here, and the loads cannot cross the fence)
#pragma unroll
        for (int px = 0; px < PX; ++px)
#pragma unroll
            for (int e = 0; e < VE; ++e) asm volatile("" : "+v"(acc[px][e]));
        asm volatile("" ::: "memory");
    }
    char* o = static_cast<char*>(d) + ((img * H + hy) * (int64_t)W * C + c0) * s;
#pragma unroll
    for (int px = 0; px < PX; ++px)
        if (wx0 + px < W) store_vals<DT, VE>(o + (int64_t)(wx0 + px) * C * s, acc[px]);
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
    int64_t pix;
    int ch;
    split_index(i, chunks, narrow_grid(), pix, ch);
    const int c0 = ch * VE;
    const int64_t at = (pix * C + c0) * s;
    float yv[VE], xv[VE];
    load_vals<DT, VE>(static_cast<const char*>(y) + at, yv);
    load_vals<DT, VE>(static_cast<const char*>(xn) + at, xv);
    const typename E::S* lg = static_cast<const typename E::S*>(rows) + pix * rstride + gate0;
    // one sigmoid per group met (a chunk of VE channels usually lies in one)
    int gprev = -1;
    float sg = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) {
        const int g = (c0 + e) / Cg;
        if (g != gprev) {
            const float t = E::to_f(lg[g]);
            sg = 1.0f / (1.0f + expf(-t));
            gprev = g;
        }
        yv[e] = yv[e] * (1.0f - sg) + xv[e] * sg;
    }
    store_vals<DT, VE>(static_cast<char*>(out) + at, yv);
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// out = a @ w^T + bias (rows of lda / ldo elements), rounded once: the vector
// kernel when the operands allow it (16-byte aligned rows and pointers,
// K * s a multiple of 16 and at most 640 bytes), else k_gemm.
template <int DT>
bool gemm_vector_ok(const void* a, int64_t lda, const void* w, const void* out, int64_t ldo, int K)
{
    constexpr int s = Elem<DT>::kBytes;
    const int64_t kb = (int64_t)K * s;
    return kb % 16 == 0 && kb <= 640 && (lda * s) % 16 == 0 && (ldo * s) % 16 == 0 && (uintptr_t)a % 16 == 0 &&
           (uintptr_t)w % 16 == 0 && (uintptr_t)out % 16 == 0;
}

// The gate can ride on the projection: vector kernel, rows of at most 256
// bytes (wider ones need more registers than the gated form has), and each
// 16-byte vector within one group.
template <int DT>
bool gemm_gate_ok(const void* a, int64_t lda, const void* w, const void* out, int64_t ldo, int K, int Cg)
{
    return gemm_vector_ok<DT>(a, lda, w, out, ldo, K) && (int64_t)K * Elem<DT>::kBytes <= 256 &&
           Cg % kPerVec<DT> == 0;
}

// gate (optional): apply the centre-feature gate to the rows as they are
// read (the caller checks gemm_gate_ok).
template <int DT>
void gemm(const void* a, int64_t lda, const void* w, const float* bias, void* out, int64_t ldo, int64_t M, int K,
          int Nn, int cus, hipStream_t st, const GateSrc* gate = nullptr)
{
    constexpr int s = Elem<DT>::kBytes;
    const int64_t kb = (int64_t)K * s;
    const bool vec = gemm_vector_ok<DT>(a, lda, w, out, ldo, K);
    if (!vec || M == 0) {
        if (M > 0)
            hipLaunchKernelGGL(k_gemm<DT>, dim3((unsigned)cdiv(M, 64)), dim3(256), 0, st, a, lda, w, bias, out, ldo,
                               M, K, Nn);
        return;
    }
    const int kv = kb <= 128 ? 2 : kb <= 256 ? 4 : 10;
    const int wpitch = (int)((kv * 64 + 127) / 128 * 128 + 16);
    // columns per pass: at most 160, and the weights plus 8 output tiles in 160 KiB
    const int ldsmax = 160 * 1024;
    int nbmax = (ldsmax - kGemmvWaves * 16 * 16) / (wpitch + kGemmvWaves * 16 * s) / 16 * 16;
    nbmax = nbmax > 16 * kGemmvMaxBlocks ? 16 * kGemmvMaxBlocks : nbmax;
    const int passes = (int)cdiv(Nn, nbmax);
    const int NB = (int)cdiv(cdiv(Nn, passes), 16) * 16;
    const int lds = NB * wpitch + kGemmvWaves * 16 * (NB * s + 16);
    const int64_t T = cdiv(M, 128);
    const int per_cu = kv == 10 ? 1 : 2;
    const int64_t gr = std::max<int64_t>(1, std::min<int64_t>(T, (int64_t)cus * per_cu / passes));
    const dim3 grid((unsigned)(gr * passes)), block(64 * kGemmvWaves);
    const GateSrc gs = gate ? *gate : GateSrc{nullptr, nullptr, 0, 0, 1};
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, grid, block, lds, st, a, lda, w, bias, out, ldo, M, K, Nn, NB, passes, wpitch, gs);
    };
    if (gate) {
        if (kv == 2) go(k_gemmv<DT, 2, 1>);
        else go(k_gemmv<DT, 4, 1>);   // (kv <= 4: gemm_gate_ok)
    } else {
        if (kv == 2) go(k_gemmv<DT, 2, 0>);
        else if (kv == 4) go(k_gemmv<DT, 4, 0>);
        else go(k_gemmv<DT, 10, 0>);
    }
}

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
    // elementwise steps: one 16-byte vector per thread when the channels
    // split into whole vectors (the workspace regions are 256-byte aligned)
    constexpr int VE = kPerVec<DT>;
    const bool vec = C % VE == 0 && (uintptr_t)m.out % 16 == 0;
    // 1. projection
    gemm<DT>(m.x_in, (int64_t)m.Cin, m.w.w_in, m.w.b_in, xp, (int64_t)C, npix, m.Cin, C, m.cus, st);
    // 2. normalisation
    if (m.norm == DCNV4_NORM_GROUP) {
        double* part = reinterpret_cast<double*>(ws + L.stats);
        float* stat = reinterpret_cast<float*>(ws + L.stats + L.stat_offset);
        if (C % VE == 0)
            hipLaunchKernelGGL((k_gn_partial<DT, VE>), dim3((unsigned)(m.N * L.slices)), dim3(256), 0, st, xp, part,
                               HW, C, L.slices);
        else
            hipLaunchKernelGGL((k_gn_partial<DT, 1>), dim3((unsigned)(m.N * L.slices)), dim3(256), 0, st, xp, part,
                               HW, C, L.slices);
        hipLaunchKernelGGL(k_gn_finalize, dim3((unsigned)cdiv((int64_t)m.N * m.norm_groups, 4)), dim3(256), 0, st,
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
        // the vector kernel addresses the whole tensor with 31-bit offsets
        const bool small = (int64_t)npix * C * (int64_t)sizeof(typename Elem<DT>::S) < ((int64_t)1 << 31);
        const unsigned grid = (unsigned)cdiv(npix * (vec ? C / VE : C), 256);
        constexpr int PX = 4;
        if (vec && lw && small)
            hipLaunchKernelGGL((k_dw3x3v<DT, PX>), dim3((unsigned)cdiv((int64_t)m.N * m.H * cdiv(m.W, PX) * (C / VE),
                                                                       256)),
                               dim3(256), wbytes, st, xn, d, m.w.w_dw, m.w.b_dw, m.N, m.H, m.W, C);
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
    gemm<DT>(d, (int64_t)C, m.w.w_pred, m.w.b_pred, rows, L.rows_stride, npix, C, L.R, m.cus, st);
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
    // 6. centre-feature gate, 7. output projection: the gate is applied by the
    // projection as it reads its rows when the vector kernel takes it (each
    // 16-byte vector within one group), else by k_gate into the workspace
    void* last = y;
    const bool fuse = m.center_scale && m.out_proj &&
                      gemm_gate_ok<DT>(y, (int64_t)C, m.w.w_out, m.out, (int64_t)m.Cout, C, m.Cg);
    if (fuse) {
        const GateSrc gs{xn, rows, L.rows_stride, 3 * m.G * L.P, m.Cg};
        gemm<DT>(y, (int64_t)C, m.w.w_out, m.w.b_out, m.out, (int64_t)m.Cout, npix, C, m.Cout, m.cus, st, &gs);
        return hipGetLastError();
    }
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
        gemm<DT>(last, (int64_t)C, m.w.w_out, m.w.b_out, m.out, (int64_t)m.Cout, npix, C, m.Cout, m.cus, st);
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

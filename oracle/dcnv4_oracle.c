/*
 * DCNv4 spatial-aggregation forward: CPU ORACLE.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it.  It shares no code, header, table or helper with the HIP
 * library; it is plain, slow, single-threaded C.
 *
 * What it computes (sources, all web pages on DCNv4):
 *   [A] "不只是卷积的平替：我把DCNv4塞进Stable Diffusion的U-Net里"
 *       (jsqmd.com/news/933833), section 1, code example "DCNv4核心计算流程示例
 *       （简化版）": for every output pixel and group, K*K points are placed on
 *       the regular grid plus a learned offset, the input is bilinearly
 *       sampled at each point, each sample is multiplied by its dynamic weight
 *       and the samples are summed over the points.  Offsets are laid out per
 *       group as (2, K*K), the weights per group as (K*K); output channel
 *       g*Cg + c comes from input channel g*Cg + c (no channel mixing).
 *   [A] section 1, first optimisation, and [B] "DCNv4：重塑视觉模型核心，三倍速率
 *       的动态稀疏卷积如何炼成？" (bqwf.cn/news/1148139) section 2.1: the
 *       dynamic weights are used raw -- no softmax, they may be negative or
 *       exceed 1.
 *   [C] "掌握DCNv4技术：3倍速度提升与80%加速效果的实战指南"
 *       (pwwt.cn/news/2159231), section "进阶优化建议": the offset_scale factor
 *       and the option that drops the centre sampling point.
 *
 * Readings where the pages are silent (each one is listed with its reason in
 * the design notes of the repository):
 *   - layout channels-last: x[N,H,W,G*Cg], out[N,Ho,Wo,G*Cg]; offsets and
 *     weights belong to OUTPUT pixels: offset[n,ho,wo, g, {x,y}, P],
 *     mask[n,ho,wo, g, P], each pixel's row at a caller-given element stride;
 *   - plane 0 of the offsets moves along W (x), plane 1 along H (y);
 *   - points enumerated row-major, k = i*K + j, i the row (H) index; with
 *     remove_center the centre (K/2, K/2) is skipped and P = K*K - 1;
 *   - base grid: ordinary convolution arithmetic with stride, pad, dilation;
 *     Ho = (H + 2*pad - dil*(K-1) - 1)/stride + 1;
 *   - sample position p = base + offset_scale * offset;
 *   - zero padding: a bilinear corner outside the image reads 0;
 *   - bilinear corners are floor(p) and floor(p)+1 (floor, not truncation).
 *
 * Two entry points:
 *   dcnv4_oracle_forward_f64  -- the plain definition in double precision.
 *   dcnv4_oracle_forward_f32  -- one fixed IEEE binary32 operation sequence
 *       (round to nearest even, no contraction except the explicit fmaf, no
 *       flush of subnormals), followed by one round-to-nearest-even into the
 *       I/O type.  The pages state that half precision is used but not how
 *       the arithmetic is ordered; this is the sequence the GPU path is
 *       compared with element by element:
 *         px = fmaf(dx, offset_scale, (float)(wo*stride - pad + j*dil))
 *         py = fmaf(dy, offset_scale, (float)(ho*stride - pad + i*dil))
 *         skip the point unless -1 < px < W and -1 < py < H (NaN skips too)
 *         fx = floorf(px); lx = px - fx; hx = 1 - lx   (same for y)
 *         mhy = m*hy; mly = m*ly
 *         w00 = mhy*hx; w01 = mhy*lx; w10 = mly*hx; w11 = mly*lx
 *         per channel, corners in the order 00, 01, 10, 11:
 *           acc = fmaf(w_ab, v_ab, acc), v_ab = 0 outside the image
 *       accumulating over points in enumeration order, acc starting at +0.
 *
 *   dcnv4_oracle_backward_f64 -- the gradients of the plain definition
 *       (triangle-kernel form, below) with respect to x, the offsets and the
 *       weights, in double precision, written out from the derivative of
 *       each factor.  The pages name the backward step only as what training
 *       needs ("不只是卷积的平替" section 4, training; the usage guide's
 *       module wraps a differentiable op); the derivative itself follows from
 *       the forward's definition.  Reading where the definition has a kink
 *       (an integer coordinate, where the bilinear corners change): the
 *       derivative from the right, which is the one that belongs to the
 *       corners floor(p) and floor(p)+1 that the forward uses.  Points the
 *       forward skips have zero gradient.  With f32_positions the sampling
 *       positions are the forward's binary32 ones (one fmaf, as in the
 *       sequence above) and everything after them is double: the reference
 *       for a binary32 evaluation of the gradients, whose positions carry
 *       that rounding by construction.
 *
 *   dcnv4_oracle_softmax_rows_f64 -- DCNv3's weight normalisation, which
 *       DCNv4 removes ("不只是卷积的平替" section 1, first optimisation;
 *       "DCNv4：重塑视觉模型核心" section 2.1; the usage guide's principle
 *       section): a softmax over the sampling points of each (pixel, group),
 *       so the weights are positive and sum to one.  Reading: the softmax
 *       runs over all P points of the group, including points that fall
 *       outside the image.  Feeding its output to the forward above gives
 *       the DCNv3-style aggregation on the same sampling.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };
enum { OR_OK = 0, OR_ERR_ARG = 1, OR_ERR_NOMEM = 2 };

/* ------------------------------------------------------------------------ */
/* Number formats, from the IEEE 754 binary16 definition and from bfloat16  */
/* (the upper 16 bits of binary32: 1 sign, 8 exponent, 7 fraction bits).   */
/* ------------------------------------------------------------------------ */

/* binary16: sign(1) exponent(5, bias 15) fraction(10). */
float dcnv4_oracle_f16_to_f32(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1f;
    const int f = h & 0x3ff;
    float v;
    if (e == 0x1f)
        v = f ? NAN : INFINITY;
    else if (e == 0)
        v = ldexpf((float)f, -24);                 /* subnormal: f * 2^-24 */
    else
        v = ldexpf((float)(1024 + f), e - 25);     /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: sign(1) exponent(8, bias 127) fraction(7). */
float dcnv4_oracle_bf16_to_f32(uint16_t b)
{
    const int sign = (b >> 15) & 1;
    const int e = (b >> 7) & 0xff;
    const int f = b & 0x7f;
    float v;
    if (e == 0xff)
        v = f ? NAN : INFINITY;
    else if (e == 0)
        v = ldexpf((float)f, -133);                /* subnormal: f * 2^-133 */
    else
        v = ldexpf((float)(128 + f), e - 134);     /* (1 + f/128) * 2^(e-127) */
    return sign ? -v : v;
}

/*
 * Round a binary32 value to a format with `mbits` fraction bits, exponent
 * bias `bias` and largest biased exponent `emax_biased` (all-ones is Inf/NaN),
 * round to nearest, ties to even.  Works on the exact value in double:
 * scaling by powers of two and nearbyint() (default rounding mode: to nearest
 * even) are exact there.
 */
static uint16_t round_to_small_float(float fin, int mbits, int ebits, int bias)
{
    const int emax_biased = (1 << ebits) - 1;
    const uint16_t sign = signbit(fin) ? (uint16_t)(1u << (mbits + ebits)) : 0;
    const uint16_t inf_bits = (uint16_t)(emax_biased << mbits);
    if (isnan(fin))
        return (uint16_t)(sign | inf_bits | (1u << (mbits - 1)));   /* quiet NaN */
    double a = fabs((double)fin);
    if (isinf(fin))
        return (uint16_t)(sign | inf_bits);
    if (a == 0.0)
        return sign;
    const int emin = 1 - bias;                       /* smallest normal exponent */
    int e2;
    frexp(a, &e2);                                   /* a = m * 2^e2, m in [0.5,1) */
    int e = e2 - 1;                                  /* a in [2^e, 2^(e+1)) */
    if (e < emin) {
        /* subnormal range: multiples of 2^(emin - mbits) */
        double q = nearbyint(ldexp(a, mbits - emin));
        /* q == 2^mbits rolls over into the smallest normal, same bit pattern */
        return (uint16_t)(sign | (uint16_t)q);
    }
    double q = nearbyint(ldexp(a, mbits - e));       /* in [2^mbits, 2^(mbits+1)] */
    if (q == ldexp(1.0, mbits + 1)) {
        q = ldexp(1.0, mbits);
        e += 1;
    }
    if (e + bias >= emax_biased)
        return (uint16_t)(sign | inf_bits);          /* overflow to infinity */
    return (uint16_t)(sign | (uint16_t)((e + bias) << mbits) |
                      (uint16_t)(q - ldexp(1.0, mbits)));
}

uint16_t dcnv4_oracle_f32_to_f16(float f) { return round_to_small_float(f, 10, 5, 15); }
uint16_t dcnv4_oracle_f32_to_bf16(float f) { return round_to_small_float(f, 7, 8, 127); }

/* Array forms, so tests can sweep whole code spaces in one call. */
void dcnv4_oracle_f16_to_f32_array(const uint16_t* in, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = dcnv4_oracle_f16_to_f32(in[i]);
}
void dcnv4_oracle_bf16_to_f32_array(const uint16_t* in, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = dcnv4_oracle_bf16_to_f32(in[i]);
}
void dcnv4_oracle_f32_to_f16_array(const float* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = dcnv4_oracle_f32_to_f16(in[i]);
}
void dcnv4_oracle_f32_to_bf16_array(const float* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = dcnv4_oracle_f32_to_bf16(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Shapes                                                                   */
/* ------------------------------------------------------------------------ */

/* Output size of ordinary convolution arithmetic; <= 0 when no output. */
int dcnv4_oracle_output_dim(int in, int K, int stride, int pad, int dil)
{
    if (in < 1 || K < 1 || stride < 1 || pad < 0 || dil < 1) return 0;
    int64_t span = (int64_t)in + 2 * (int64_t)pad - (int64_t)dil * (K - 1) - 1;
    if (span < 0) return 0;
    return (int)(span / stride + 1);
}

typedef struct {
    int N, H, W, G, Cg, K, stride, pad, dil, remove_center;
    int Ho, Wo, P;
    int64_t off_stride, mask_stride;   /* elements between output pixels */
} shape_t;

static int make_shape(shape_t* s, int N, int H, int W, int G, int Cg, int K,
                      int stride, int pad, int dil, int remove_center,
                      int64_t off_stride, int64_t mask_stride)
{
    if (N < 0 || H < 1 || W < 1 || G < 1 || Cg < 1 || K < 1) return OR_ERR_ARG;
    if (remove_center && (K % 2 == 0 || K == 1)) return OR_ERR_ARG;
    s->N = N; s->H = H; s->W = W; s->G = G; s->Cg = Cg; s->K = K;
    s->stride = stride; s->pad = pad; s->dil = dil;
    s->remove_center = remove_center ? 1 : 0;
    s->Ho = dcnv4_oracle_output_dim(H, K, stride, pad, dil);
    s->Wo = dcnv4_oracle_output_dim(W, K, stride, pad, dil);
    if (s->Ho < 1 || s->Wo < 1) return OR_ERR_ARG;
    s->P = K * K - s->remove_center;
    s->off_stride = off_stride > 0 ? off_stride : (int64_t)G * 2 * s->P;
    s->mask_stride = mask_stride > 0 ? mask_stride : (int64_t)G * s->P;
    return OR_OK;
}

/* Convert n elements of the I/O type to binary32 (exact for f16 and bf16). */
static float* to_f32_copy(const void* src, int64_t n, int dtype)
{
    float* dst = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    if (!dst) return NULL;
    if (dtype == OR_F32) {
        memcpy(dst, src, (size_t)n * sizeof(float));
    } else if (dtype == OR_F16) {
        dcnv4_oracle_f16_to_f32_array((const uint16_t*)src, dst, n);
    } else {
        dcnv4_oracle_bf16_to_f32_array((const uint16_t*)src, dst, n);
    }
    return dst;
}

/* ------------------------------------------------------------------------ */
/* The operator, binary32 operation sequence (comparison oracle)           */
/* ------------------------------------------------------------------------ */

int dcnv4_oracle_forward_f32(const void* x, const void* offset, const void* mask, void* out,
                             int N, int H, int W, int G, int Cg, int K,
                             int stride, int pad, int dil, float offset_scale,
                             int remove_center, int64_t off_stride, int64_t mask_stride,
                             int dtype)
{
    shape_t s;
    if (dtype < OR_F32 || dtype > OR_BF16) return OR_ERR_ARG;
    if (make_shape(&s, N, H, W, G, Cg, K, stride, pad, dil, remove_center,
                   off_stride, mask_stride) != OR_OK)
        return OR_ERR_ARG;
    if (N == 0) return OR_OK;
    const int64_t C = (int64_t)G * Cg;
    const int64_t npix_out = (int64_t)N * s.Ho * s.Wo;
    const int64_t n_x = (int64_t)N * H * W * C;
    /* the last pixel's row only needs to reach its last used element */
    const int64_t n_off = (npix_out - 1) * s.off_stride + (int64_t)G * 2 * s.P;
    const int64_t n_mask = (npix_out - 1) * s.mask_stride + (int64_t)G * s.P;

    float* xf = to_f32_copy(x, n_x, dtype);
    float* of = to_f32_copy(offset, n_off, dtype);
    float* mf = to_f32_copy(mask, n_mask, dtype);
    float* acc = (float*)malloc((size_t)Cg * sizeof(float));
    if (!xf || !of || !mf || !acc) {
        free(xf); free(of); free(mf); free(acc);
        return OR_ERR_NOMEM;
    }

    for (int n = 0; n < N; ++n)
    for (int ho = 0; ho < s.Ho; ++ho)
    for (int wo = 0; wo < s.Wo; ++wo) {
        const int64_t pix = ((int64_t)n * s.Ho + ho) * s.Wo + wo;
        for (int g = 0; g < G; ++g) {
            const float* dxs = of + pix * s.off_stride + (int64_t)g * 2 * s.P;
            const float* dys = dxs + s.P;
            const float* ms = mf + pix * s.mask_stride + (int64_t)g * s.P;
            for (int c = 0; c < Cg; ++c) acc[c] = 0.0f;
            int k = 0;
            for (int i = 0; i < K; ++i)
            for (int j = 0; j < K; ++j) {
                if (s.remove_center && i == K / 2 && j == K / 2) continue;
                const float dx = dxs[k], dy = dys[k], m = ms[k];
                ++k;
                const float px = fmaf(dx, offset_scale, (float)(wo * stride - pad + j * dil));
                const float py = fmaf(dy, offset_scale, (float)(ho * stride - pad + i * dil));
                if (!(px > -1.0f && px < (float)W && py > -1.0f && py < (float)H))
                    continue;
                const float fx = floorf(px), fy = floorf(py);
                const int x0 = (int)fx, y0 = (int)fy;
                const float lx = px - fx, ly = py - fy;
                const float hx = 1.0f - lx, hy = 1.0f - ly;
                const float mhy = m * hy, mly = m * ly;
                const float wgt[2][2] = { { mhy * hx, mhy * lx }, { mly * hx, mly * lx } };
                for (int c = 0; c < Cg; ++c) {
                    for (int a = 0; a < 2; ++a)
                    for (int b = 0; b < 2; ++b) {
                        const int yy = y0 + a, xx = x0 + b;
                        float v = 0.0f;
                        if (yy >= 0 && yy < H && xx >= 0 && xx < W)
                            v = xf[(((int64_t)n * H + yy) * W + xx) * C + (int64_t)g * Cg + c];
                        acc[c] = fmaf(wgt[a][b], v, acc[c]);
                    }
                }
            }
            const int64_t obase = pix * C + (int64_t)g * Cg;
            for (int c = 0; c < Cg; ++c) {
                if (dtype == OR_F32)
                    ((float*)out)[obase + c] = acc[c];
                else if (dtype == OR_F16)
                    ((uint16_t*)out)[obase + c] = dcnv4_oracle_f32_to_f16(acc[c]);
                else
                    ((uint16_t*)out)[obase + c] = dcnv4_oracle_f32_to_bf16(acc[c]);
            }
        }
    }
    free(xf); free(of); free(mf); free(acc);
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* The operator, plain definition in double precision                       */
/* ------------------------------------------------------------------------ */

/*
 * out = sum over points of m * Bilinear(x, p), p = base + offset_scale*offset,
 * Bilinear(f, p) = sum over the (at most four) integer pixels q with
 * |p - q| < 1 per axis, inside the image, of (1-|py-qy|)(1-|px-qx|) f(q).
 * The range test only guards the float->int conversion: a point outside
 * (-1,H) x (-1,W) has no pixel inside the image with nonzero weight.
 */
int dcnv4_oracle_forward_f64(const double* x, const double* offset, const double* mask,
                             double* out, int N, int H, int W, int G, int Cg, int K,
                             int stride, int pad, int dil, double offset_scale,
                             int remove_center, int64_t off_stride, int64_t mask_stride)
{
    shape_t s;
    if (make_shape(&s, N, H, W, G, Cg, K, stride, pad, dil, remove_center,
                   off_stride, mask_stride) != OR_OK)
        return OR_ERR_ARG;
    const int64_t C = (int64_t)G * Cg;
    for (int n = 0; n < N; ++n)
    for (int ho = 0; ho < s.Ho; ++ho)
    for (int wo = 0; wo < s.Wo; ++wo) {
        const int64_t pix = ((int64_t)n * s.Ho + ho) * s.Wo + wo;
        for (int g = 0; g < G; ++g) {
            double* o = out + pix * C + (int64_t)g * Cg;
            for (int c = 0; c < Cg; ++c) o[c] = 0.0;
            int k = 0;
            for (int i = 0; i < K; ++i)
            for (int j = 0; j < K; ++j) {
                if (s.remove_center && i == K / 2 && j == K / 2) continue;
                const double dx = offset[pix * s.off_stride + (int64_t)g * 2 * s.P + k];
                const double dy = offset[pix * s.off_stride + (int64_t)g * 2 * s.P + s.P + k];
                const double m = mask[pix * s.mask_stride + (int64_t)g * s.P + k];
                ++k;
                const double px = (double)(wo * stride - pad + j * dil) + offset_scale * dx;
                const double py = (double)(ho * stride - pad + i * dil) + offset_scale * dy;
                if (!(px > -1.0 && px < W && py > -1.0 && py < H)) continue;
                const int x0 = (int)floor(px), y0 = (int)floor(py);
                for (int qy = y0; qy <= y0 + 1; ++qy)
                for (int qx = x0; qx <= x0 + 1; ++qx) {
                    if (qy < 0 || qy >= H || qx < 0 || qx >= W) continue;
                    const double wgt = (1.0 - fabs(py - qy)) * (1.0 - fabs(px - qx));
                    const double* xv = x + (((int64_t)n * H + qy) * W + qx) * C + (int64_t)g * Cg;
                    for (int c = 0; c < Cg; ++c) o[c] += m * wgt * xv[c];
                }
            }
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Gradients of the plain definition (double precision)                    */
/* ------------------------------------------------------------------------ */

/* Triangle kernel and its derivative from the right:
 *   tri(t) = max(0, 1 - |t|);  dtri(t) = -1 for 0 <= t < 1, +1 for -1 <= t < 0,
 * 0 elsewhere.  A sample at p is sum_q tri(py - qy) tri(px - qx) f(q) over the
 * integer pixels q of the image, so
 *   d sample / d f(q) = tri(py - qy) tri(px - qx)
 *   d sample / d px   = sum_q tri(py - qy) dtri(px - qx) f(q)
 *   d sample / d py   = sum_q dtri(py - qy) tri(px - qx) f(q)
 * and out = sum_k m_k sample_k, with p_k = base_k + offset_scale * offset_k. */
static double tri(double t) { t = fabs(t); return t < 1.0 ? 1.0 - t : 0.0; }
static double dtri(double t)
{
    if (t >= 0.0 && t < 1.0) return -1.0;
    if (t >= -1.0 && t < 0.0) return 1.0;
    return 0.0;
}

/*
 * grad_out [N,Ho,Wo,G*Cg]; outputs (all double, overwritten):
 *   grad_x      [N,H,W,G*Cg]
 *   grad_offset rows of off_stride elements per output pixel (G,2,P used)
 *   grad_mask   rows of mask_stride elements per output pixel (G,P used)
 * Optional (may be NULL), for error bounds of a binary32 evaluation:
 *   abs_x       [N,H,W,G*Cg]  sum of |term| over the terms of grad_x
 *   cnt_x       [N,H,W,G*Cg]  number of terms of grad_x
 *   abs_offset  like grad_offset: sum over c and the two corners of each
 *               difference of |g_c| * weight * (|f(q1)| + |f(q0)|), times |m * scale|
 *   abs_mask    like grad_mask: sum of |g_c * weight * f(q)|
 */
int dcnv4_oracle_backward_f64(const double* x, const double* offset, const double* mask,
                              const double* grad_out, double* grad_x, double* grad_offset,
                              double* grad_mask, double* abs_x, double* cnt_x, double* abs_offset,
                              double* abs_mask, int N, int H, int W, int G, int Cg, int K,
                              int stride, int pad, int dil, double offset_scale,
                              int remove_center, int64_t off_stride, int64_t mask_stride,
                              int f32_positions)
{
    shape_t s;
    if (make_shape(&s, N, H, W, G, Cg, K, stride, pad, dil, remove_center,
                   off_stride, mask_stride) != OR_OK)
        return OR_ERR_ARG;
    const int64_t C = (int64_t)G * Cg;
    const int64_t nx = (int64_t)N * H * W * C;
    for (int64_t i = 0; i < nx; ++i) {
        grad_x[i] = 0.0;
        if (abs_x) abs_x[i] = 0.0;
        if (cnt_x) cnt_x[i] = 0.0;
    }
    for (int n = 0; n < N; ++n)
    for (int ho = 0; ho < s.Ho; ++ho)
    for (int wo = 0; wo < s.Wo; ++wo) {
        const int64_t pix = ((int64_t)n * s.Ho + ho) * s.Wo + wo;
        for (int g = 0; g < G; ++g) {
            const double* go = grad_out + pix * C + (int64_t)g * Cg;
            double* gox = grad_offset + pix * s.off_stride + (int64_t)g * 2 * s.P;
            double* gm = grad_mask + pix * s.mask_stride + (int64_t)g * s.P;
            int k = 0;
            for (int i = 0; i < K; ++i)
            for (int j = 0; j < K; ++j) {
                if (s.remove_center && i == K / 2 && j == K / 2) continue;
                const double dx = offset[pix * s.off_stride + (int64_t)g * 2 * s.P + k];
                const double dy = offset[pix * s.off_stride + (int64_t)g * 2 * s.P + s.P + k];
                const double m = mask[pix * s.mask_stride + (int64_t)g * s.P + k];
                double px = (double)(wo * stride - pad + j * dil) + offset_scale * dx;
                double py = (double)(ho * stride - pad + i * dil) + offset_scale * dy;
                if (f32_positions) {
                    px = (double)fmaf((float)dx, (float)offset_scale, (float)(wo * stride - pad + j * dil));
                    py = (double)fmaf((float)dy, (float)offset_scale, (float)(ho * stride - pad + i * dil));
                }
                double d_px = 0.0, d_py = 0.0, d_m = 0.0, a_px = 0.0, a_py = 0.0, a_m = 0.0;
                if (px > -1.0 && px < W && py > -1.0 && py < H) {
                    const int x0 = (int)floor(px), y0 = (int)floor(py);
                    for (int qy = y0; qy <= y0 + 1; ++qy)
                    for (int qx = x0; qx <= x0 + 1; ++qx) {
                        if (qy < 0 || qy >= H || qx < 0 || qx >= W) continue;
                        const double ty = tri(py - qy), tx = tri(px - qx);
                        const double sy = dtri(py - qy), sx = dtri(px - qx);
                        const int64_t q = (((int64_t)n * H + qy) * W + qx) * C + (int64_t)g * Cg;
                        for (int c = 0; c < Cg; ++c) {
                            const double f = x[q + c];
                            grad_x[q + c] += m * ty * tx * go[c];
                            if (abs_x) abs_x[q + c] += fabs(m * ty * tx * go[c]);
                            if (cnt_x) cnt_x[q + c] += 1.0;
                            d_m += go[c] * ty * tx * f;
                            d_px += go[c] * ty * sx * f;
                            d_py += go[c] * sy * tx * f;
                            a_m += fabs(go[c] * ty * tx * f);
                            a_px += fabs(go[c] * ty * f);
                            a_py += fabs(go[c] * tx * f);
                        }
                    }
                }
                gm[k] = d_m;
                gox[k] = offset_scale * m * d_px;
                gox[s.P + k] = offset_scale * m * d_py;
                if (abs_mask) abs_mask[pix * s.mask_stride + (int64_t)g * s.P + k] = a_m;
                if (abs_offset) {
                    abs_offset[pix * s.off_stride + (int64_t)g * 2 * s.P + k] = fabs(offset_scale * m) * a_px;
                    abs_offset[pix * s.off_stride + (int64_t)g * 2 * s.P + s.P + k] = fabs(offset_scale * m) * a_py;
                }
                ++k;
            }
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* DCNv3-style weights: softmax over each group's P points (double)        */
/* ------------------------------------------------------------------------ */

/* mask: nrows rows of `stride` elements, G groups of P weights each at the
 * start of a row; out: the same layout (only the G*P weights written).
 * exp(m_k - max_j m_j) / sum_j exp(m_j - max_j m_j): the usual shifted form,
 * equal to exp(m_k) / sum_j exp(m_j) and free of overflow. */
int dcnv4_oracle_softmax_rows_f64(const double* mask, double* out, int64_t nrows, int G, int P,
                                  int64_t stride)
{
    if (nrows < 0 || G < 1 || P < 1 || stride < (int64_t)G * P) return OR_ERR_ARG;
    for (int64_t r = 0; r < nrows; ++r)
        for (int g = 0; g < G; ++g) {
            const double* m = mask + r * stride + (int64_t)g * P;
            double* o = out + r * stride + (int64_t)g * P;
            double mx = m[0];
            for (int k = 1; k < P; ++k) mx = m[k] > mx ? m[k] : mx;
            double sum = 0.0;
            for (int k = 0; k < P; ++k) sum += exp(m[k] - mx);
            for (int k = 0; k < P; ++k) o[k] = exp(m[k] - mx) / sum;
        }
    return OR_OK;
}

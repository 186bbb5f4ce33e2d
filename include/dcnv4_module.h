/*
 * dcnv4_module.h -- C ABI of the DCNv4 module forward in libdcnv4.so: the
 * steps around the spatial-aggregation operator of dcnv4.h, on AMD Instinct
 * MI355X (gfx950).
 *
 * The module (web pages on DCNv4):
 *   "不只是卷积的平替：我把DCNv4塞进Stable Diffusion的U-Net里" (jsqmd.com/news/933833),
 *   section 2, the DCNv4Block example and item 2 of the list before it: a 1x1
 *   convolution adjusts the channels, a normalisation follows (the example
 *   uses a group norm, the list a layer norm: both are offered), and ONE
 *   predictor produces the offsets and the dynamic weights together -- a
 *   depthwise 3x3 convolution (padding 1) and a 1x1 convolution to 3*G*P
 *   channels, no activation and no further normalisation between them; the
 *   first 2*G*P channels are the offsets (per group: the P x-offsets, then
 *   the P y-offsets), the next G*P the weights (per group, P raw weights).
 *   The operator (dcnv4.h, K = 3, stride 1, padding 1, dilation 1) samples
 *   the normalised features.
 *   "掌握DCNv4技术：3倍速度提升与80%加速效果的实战指南" (pwwt.cn/news/2159231),
 *   section "进阶优化建议": centre-feature scaling through a sigmoid, and an
 *   option that drops the centre point (P = 8 instead of 9).
 *
 * Steps, channels-last [N, H, W, .] throughout (C = G * Cg):
 *   1. xp   = x_in @ w_in^T + b_in                      [N,H,W,C]   (1x1 conv)
 *   2. xn   = norm(xp) * gamma + beta                   [N,H,W,C]
 *             group norm: mean and biased variance per (image, channel group)
 *             over H, W and the group's channels; layer norm: per pixel over C;
 *             (v - mean) / sqrt(var + eps); or no normalisation (xn = xp)
 *   3. d    = depthwise3x3(xn) + b_dw                   [N,H,W,C]   (zero padding 1;
 *             w_dw[c][i][j] multiplies xn[h + i - 1][w + j - 1][c])
 *   4. rows = d @ w_pred^T + b_pred                     [N,H,W,R]
 *             R = 3*G*P, plus G gate logits when centre scaling is on
 *   5. y    = dcnv4 operator(xn, offsets = rows[.., 0:2GP], weights = rows[.., 2GP:3GP])
 *   6. centre scaling (optional): s = sigmoid(rows[.., 3GP + g]) per group g,
 *             y = y * (1 - s) + xn * s   (the pixel's own normalised feature)
 *   7. out  = y @ w_out^T + b_out (optional output projection, Cout channels),
 *             else out = y (Cout = C)
 * With both 6 and 7, the gate is applied while the projection reads its
 * rows -- the same operations and rounding, the gated rows not stored --
 * when C * s <= 256 bytes, Cg * s is a multiple of 16 and out and w_out are
 * 16-byte aligned (s = bytes per element); otherwise the gated rows go to
 * the workspace first.
 * Each step's result is rounded once to the I/O type (nearest even) and read
 * back as such by the next step; arithmetic inside a step is binary32 (the
 * normalisation statistics binary64).  Step 5 is the operator of dcnv4.h,
 * bit for bit, on the stored xn and rows.
 *
 * Weights: the matrices (w_in, w_pred, w_out) in the I/O type, row-major
 * [out, in]; every vector and the depthwise taps in binary32.  All pointers
 * are device pointers owned by the caller.  The intermediate tensors live in
 * a caller-owned workspace (dcnv4_module_workspace_layout gives its size and
 * layout, so that a caller may read them), which the call overwrites; the call
 * allocates nothing.  Enqueued on `stream`, no synchronisation; validation
 * before any HIP call, as in dcnv4.h.
 */
#ifndef DCNV4_MODULE_H
#define DCNV4_MODULE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dcnv4_norm {
    DCNV4_NORM_NONE = 0,
    DCNV4_NORM_GROUP = 1,   /* group norm, norm_groups groups of C / norm_groups channels */
    DCNV4_NORM_LAYER = 2    /* layer norm over the C channels of each pixel */
} dcnv4_norm;

typedef struct dcnv4_module_config {
    int Cin;              /* input channels */
    int G, Cg;            /* operator groups and channels per group, C = G * Cg */
    int Cout;             /* output channels (the output projection's; C without it) */
    int norm;             /* dcnv4_norm */
    int norm_groups;      /* group norm: number of groups, dividing C */
    float eps;            /* added to the variance, > 0 */
    int remove_center;    /* 1: P = 8 points (the centre dropped), else P = 9 */
    int center_scale;     /* 1: the sigmoid centre-feature gate (G more predictor rows) */
    int out_proj;         /* 1: output projection w_out / b_out */
    float offset_scale;   /* the operator's offset scale */
} dcnv4_module_config;

typedef struct dcnv4_module_weights {
    const void* w_in;     /* [C, Cin] I/O type */
    const float* b_in;    /* [C] */
    const float* gamma;   /* [C] (unused without normalisation) */
    const float* beta;    /* [C] */
    const float* w_dw;    /* [C, 3, 3] */
    const float* b_dw;    /* [C] */
    const void* w_pred;   /* [R, C] I/O type, R = 3*G*P (+ G with centre scaling) */
    const float* b_pred;  /* [R] */
    const void* w_out;    /* [Cout, C] I/O type (out_proj only) */
    const float* b_out;   /* [Cout] (out_proj only) */
} dcnv4_module_weights;

/* Byte offsets of the intermediates in the workspace (each 256-byte
 * aligned); a region a configuration does not use has offset -1.  Row
 * strides in elements: C for xp, xn, d, y and gated; rows_stride for rows.
 * gated (gate and output projection both on) is written only when the
 * projection does not apply the gate itself (step 6 above). */
typedef struct dcnv4_module_layout {
    int64_t xp, xn, d, rows, y, gated;  /* [N,H,W,.] in the I/O type */
    int64_t stats;                      /* group-norm statistics (binary64 partial sums, then
                                           binary32 mean and 1/sqrt(var + eps) per (image, group)) */
    int64_t rows_stride;                /* elements per pixel of rows (R rounded up to 8) */
    int64_t total;                      /* workspace bytes */
} dcnv4_module_layout;

/* Workspace layout for a problem; DCNV4_OK or a validation status. */
int dcnv4_module_workspace_layout(int N, int H, int W, const dcnv4_module_config* cfg, int dtype,
                                  dcnv4_module_layout* layout);

/*
 * The module forward: x_in [N, H, W, Cin] -> out [N, H, W, Cout] (I/O type).
 * workspace: workspace_bytes >= layout.total device bytes, 256-byte aligned,
 * overlapping neither the inputs, the weights nor out (else
 * DCNV4_ERR_ALIAS / DCNV4_ERR_TOO_LARGE).  Shapes: N >= 0, H, W, Cin, G, Cg,
 * Cout >= 1, Cin, C and Cout at most 4096, norm_groups dividing C.
 */
int dcnv4_module_forward(const void* x_in, const dcnv4_module_weights* weights, void* out,
                         int N, int H, int W, const dcnv4_module_config* cfg,
                         void* workspace, size_t workspace_bytes, int dtype, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * module forward, its intermediates held in a library-owned device array of
 * DCNV4_MODULE_SCRATCH_BYTES per GPU instead of a workspace argument.  The
 * array is part of the library's code object (each GPU the library runs on
 * holds it until the process ends); the call allocates and frees nothing.
 * A problem whose workspace (dcnv4_module_workspace_layout's total) exceeds
 * the array is rejected with DCNV4_ERR_TOO_LARGE before any HIP call.  Every
 * call on a GPU uses that GPU's one array and leaves its intermediates there
 * (no step reads a part of it that the same call has not written first):
 * calls that overlap on one GPU (two streams, two host threads) race, and
 * the caller must order them.  Other arguments and errors as for
 * dcnv4_module_forward.
 */
#define DCNV4_MODULE_SCRATCH_BYTES ((size_t)64 << 20)

int dcnv4_module_forward_noalloc(const void* x_in, const dcnv4_module_weights* weights, void* out,
                                 int N, int H, int W, const dcnv4_module_config* cfg, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DCNV4_MODULE_H */

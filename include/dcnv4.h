/*
 * dcnv4.h -- C ABI of libdcnv4.so: the DCNv4 spatial-aggregation forward on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (web pages on DCNv4):
 *   "不只是卷积的平替：我把DCNv4塞进Stable Diffusion的U-Net里" (jsqmd.com/news/933833),
 *   section 1, code example "DCNv4核心计算流程示例（简化版）": for every output
 *   pixel and group, K*K sampling points sit on the regular convolution grid
 *   moved by learned offsets; the input is bilinearly sampled at each point,
 *   each sample is multiplied by its dynamic weight, and the weighted samples
 *   are summed over the points.  Groups share nothing: output channel
 *   g*Cg + c depends only on input channel g*Cg + c.
 *   Same page, section 1, first optimisation, and "DCNv4：重塑视觉模型核心，三倍速率
 *   的动态稀疏卷积如何炼成？" (bqwf.cn/news/1148139), section 2.1: the dynamic
 *   weights are raw -- no softmax over the points; they may be negative and
 *   may exceed 1.
 *   "掌握DCNv4技术：3倍速度提升与80%加速效果的实战指南" (pwwt.cn/news/2159231),
 *   section "进阶优化建议": offset_scale scales the offsets; an option drops the
 *   centre point.
 *
 * Conventions fixed where the pages are silent:
 *   - channels-last tensors; offsets and weights belong to OUTPUT pixels;
 *   - offset row of one group = (2, P): plane 0 moves the point along W (x),
 *     plane 1 along H (y); P = K*K points enumerated row-major, k = i*K + j,
 *     i the row index (P = K*K - 1 with the centre removed, order otherwise
 *     unchanged);
 *   - point k of output pixel (ho, wo):
 *       px = wo*stride - pad + j*dilation + offset_scale * dx[k]
 *       py = ho*stride - pad + i*dilation + offset_scale * dy[k]
 *   - bilinear sampling between floor(p) and floor(p)+1 per axis; pixels
 *     outside the image read as zero; a point with px <= -1, px >= W,
 *     py <= -1 or py >= H (or a NaN coordinate) contributes nothing;
 *   - Ho = (H + 2*pad - dilation*(K-1) - 1) / stride + 1, the same for Wo.
 *
 * Arithmetic: every I/O type is widened exactly to binary32, all arithmetic
 * is binary32 (round to nearest even, subnormals kept) in this order, and the
 * result is rounded once to the I/O type (nearest even):
 *     px = fma(dx, offset_scale, (float)(wo*stride - pad + j*dilation)), py alike
 *     lx = px - floor(px), hx = 1 - lx, ly and hy alike
 *     w00 = (m*hy)*hx, w01 = (m*hy)*lx, w10 = (m*ly)*hx, w11 = (m*ly)*lx
 *     per channel, points in order, corners 00, 01, 10, 11: acc = fma(w, v, acc)
 * so results do not depend on the launch configuration, the vector width,
 * the alignment of the pointers or the stream.
 *
 * All pointers are DEVICE pointers, owned by the caller; the library keeps no
 * reference after the call returns and allocates no device memory.  Work is
 * enqueued on `stream` (a hipStream_t; NULL = the default stream) and the call
 * returns without synchronising: DCNV4_OK means "validated and launched".
 * Every argument is validated before any HIP call; on an error nothing is
 * launched and nothing is written.  Calls are thread-safe.
 */
#ifndef DCNV4_H
#define DCNV4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* I/O element type, the same for x, offset, mask and out. */
typedef enum dcnv4_dtype {
    DCNV4_F32 = 0,   /* IEEE binary32 */
    DCNV4_F16 = 1,   /* IEEE binary16 */
    DCNV4_BF16 = 2   /* bfloat16 (upper half of binary32) */
} dcnv4_dtype;

typedef enum dcnv4_status {
    DCNV4_OK = 0,
    DCNV4_ERR_NULL = 1,       /* a pointer is NULL while there is work to do */
    DCNV4_ERR_SHAPE = 2,      /* N < 0, or H, W, G or Cg < 1 */
    DCNV4_ERR_PARAM = 3,      /* K, stride, dilation < 1; pad < 0; Ho or Wo < 1;
                                 offset_scale not finite; bad remove_center or row stride */
    DCNV4_ERR_DTYPE = 4,      /* dtype not one of dcnv4_dtype */
    DCNV4_ERR_ALIAS = 5,      /* out overlaps x, offset or mask */
    DCNV4_ERR_TOO_LARGE = 6,  /* H or W >= 2^24, one image of x, out, offset or
                                 mask spanning >= 2^31 bytes, or N*Ho*Wo*G >= 2^31 */
    DCNV4_ERR_HIP = 7,        /* no gfx950 device current, or the launch failed */
    DCNV4_ERR_ALIGN = 8       /* a pointer is not aligned to the element size */
} dcnv4_status;

/*
 * The forward operator.
 *   x       [N, H, W, G*Cg]        input, channels-last, contiguous
 *   offset  [N, Ho, Wo, G*2*K*K]   per output pixel and group: K*K x-offsets then
 *                                  K*K y-offsets, in pixels, contiguous
 *   mask    [N, Ho, Wo, G*K*K]     dynamic weights, raw (no softmax), contiguous
 *   out     [N, Ho, Wo, G*Cg]      written in full; must not overlap the inputs
 * N == 0 is a valid no-op.  Returns a dcnv4_status.
 */
int dcnv4_forward(const void* x, const void* offset, const void* mask, void* out,
                  int N, int H, int W, int G, int Cg,
                  int K, int stride, int pad, int dilation, float offset_scale,
                  int dtype, void* stream);

/*
 * The same operator with the two variants the pages name
 * (pwwt.cn/news/2159231, section "进阶优化建议": dropping the centre point;
 * jsqmd.com/news/933833, section 2, DCNv4Block example: offsets and weights
 * predicted together by one projection and split per pixel):
 *   remove_center  0 or 1; 1 drops point (K/2, K/2), needs odd K >= 3, and
 *                  P = K*K - 1 points per group are read
 *   offset_row     elements from one output pixel's offsets to the next
 *                  (0 = G*2*P, dense); must be >= G*2*P
 *   mask_row       the same for the weights (0 = G*P); must be >= G*P
 * With offset = packed, mask = packed + G*2*P and both rows = G*3*P this reads
 * a packed [N, Ho, Wo, G*3*P] tensor in place.
 */
int dcnv4_forward_ex(const void* x, const void* offset, const void* mask, void* out,
                     int N, int H, int W, int G, int Cg,
                     int K, int stride, int pad, int dilation, float offset_scale,
                     int remove_center, int64_t offset_row, int64_t mask_row,
                     int dtype, void* stream);

/*
 * The DCNv3-style aggregation on the same sampling, for comparison: the
 * weights of each (pixel, group) pass through a softmax over their P points
 * before use -- the normalisation DCNv4 removes ("不只是卷积的平替"
 * (jsqmd.com/news/933833) section 1, first optimisation; bqwf.cn/news/1148139
 * section 2.1).  The softmax covers all P points, in or out of the image.
 * Arguments as dcnv4_forward_ex.  Arithmetic: mx = max_k m_k; S = sum over k
 * in order of expf(m_k - mx); w_k = expf(m_k - mx) / S (IEEE division), then
 * the operation sequence above with w_k as the weight.  expf is the device
 * library's, so results match a reference to within its error, not bit for
 * bit.  Runs on the same kernels and plans as dcnv4_forward_ex; both kernel
 * families compute the weights with the same binary32 operations and give
 * the same bits.
 */
int dcnv4_forward_softmax(const void* x, const void* offset, const void* mask, void* out,
                          int N, int H, int W, int G, int Cg,
                          int K, int stride, int pad, int dilation, float offset_scale,
                          int remove_center, int64_t offset_row, int64_t mask_row,
                          int dtype, void* stream);

/*
 * Gradients of the operator (dcnv4_forward_ex's arguments) given grad_out =
 * dL/dout [N, Ho, Wo, G*Cg] in the I/O type.  The forward is
 *   out = sum_k m_k * sum_q tri(py_k - qy) tri(px_k - qx) x[q],
 *   tri(t) = max(0, 1 - |t|),  p_k = base_k + offset_scale * offset_k,
 * (the definition of jsqmd.com/news/933833 section 1 in triangle-kernel form);
 * its derivative with respect to a position is taken from the right at
 * integer coordinates (the side whose corners floor(p), floor(p)+1 the
 * forward uses), and points the forward skips have zero gradient.
 * Gradients are binary32, whatever the I/O type:
 *   grad_x       [N, H, W, G*Cg], overwritten (zeroed, then accumulated)
 *   grad_offset  rows of offset_row elements per output pixel, like offset;
 *                only the G*2*P gradient elements of each row are written
 *   grad_mask    rows of mask_row elements, like mask; G*P elements written
 * Any gradient pointer may be NULL (not computed).  Arithmetic is binary32;
 * grad_offset and grad_mask are summed in a fixed order (reproducible).
 * grad_x: for K = 3 when a few channels of the zero-bordered image fit in
 * LDS, each term w*g (the exact product of its binary32 factors) is rounded
 * to a multiple of 2^-F and summed exactly in
 * 64-bit integers (reproducible; F per (image, group) from the largest
 * |weight| * |grad_out| and the term count, so sums cannot overflow; the
 * binary32 path if either holds a non-finite value).  Each term's rounding
 * error is then at most M * 2^-min(51, 62 - c), M = max|weight| * max|grad_out|
 * over the (image, group) and 2^c >= 4 * P * Ho * Wo: at most M * 2^-40 for
 * images with 4 * P * Ho * Wo <= 2^22 (256 x 256 outputs with K = 3).  For K = 3 and larger
 * images the same is done per 64 x 64-pixel tile (F per tile), for the units
 * whose grid centre lies within 16 pixels of the tile; terms from units
 * farther away are added with hardware atomic adds, so elements that receive
 * such terms are summed in no fixed order (environment DCNV4_BWD_TILE=
 * "<log2 side>,<margin>" changes both: side 8..128, margin 0..256).  Other
 * kernel sizes: hardware atomic adds, whose order is not fixed.  Gradients must not
 * overlap the inputs or grad_x; grad_offset and grad_mask may interleave
 * (one packed tensor) but must not share elements.  Needs Cg*s <= 64 vectors
 * of the widest width the pointers allow (else DCNV4_ERR_TOO_LARGE).
 * Validation, ownership and stream semantics as for dcnv4_forward.
 */
int dcnv4_backward(const void* x, const void* offset, const void* mask, const void* grad_out,
                   float* grad_x, float* grad_offset, float* grad_mask,
                   int N, int H, int W, int G, int Cg,
                   int K, int stride, int pad, int dilation, float offset_scale,
                   int remove_center, int64_t offset_row, int64_t mask_row,
                   int dtype, void* stream);

/* Ho or Wo for an input extent; <= 0 when the arguments admit no output. */
int dcnv4_output_dim(int in, int K, int stride, int pad, int dilation);

/* Static text for a status code ("unknown status" for anything else). */
const char* dcnv4_status_string(int status);

/* Details of the last failed call on the calling thread ("" if none). */
const char* dcnv4_last_error(void);

/* Library version, e.g. "0.1.0". */
const char* dcnv4_version(void);

/*
 * Launch plan the library would use for these arguments (for reporting and
 * tests).  Pure host computation, no HIP call.
 * The planners size grids for the device's compute units (their count is
 * read once per device at the first call on it); a plan query, which makes no
 * HIP call, assumes an MI355X's 256.  The environment variable DCNV4_CUS
 * (1..4096) overrides the count for both (tests; a partitioned device).
 */
typedef struct dcnv4_plan {
    int kernel;           /* kernel family id, see dcnv4_kernel_name */
    int vec;              /* bytes per lane per corner read (direct family) */
    int lanes_per_unit;   /* lanes sharing one (pixel, group) unit */
    int block;            /* threads per workgroup */
    int64_t grid;         /* workgroups */
    int groups_per_block; /* window family: groups staged together */
    int tile_h, tile_w;   /* window family: output tile per workgroup */
    int margin_y, margin_x; /* window family: rows/cols staged beyond the tile footprint */
    int window_h, window_w; /* window family: staged window (pixels) */
    int full_window;      /* window family: 1 if the window is the whole zero-bordered image */
    int lds_bytes;        /* LDS per workgroup (window and offset-row buffers) */
    int coalesced_offsets; /* window family: 1 if each wave stages its units' offset rows
                              through LDS with in-order loads */
    int shared_coefficients; /* window family, units split over lanes: 1 if each lane computes
                                a share of the points' positions and weights and the unit's
                                lanes exchange them (quad permutation), 0 if every lane
                                computes all of them */
} dcnv4_plan;

int dcnv4_query_plan(const void* x, const void* offset, const void* mask, const void* out,
                     int N, int H, int W, int G, int Cg,
                     int K, int stride, int pad, int dilation, float offset_scale,
                     int remove_center, int64_t offset_row, int64_t mask_row,
                     int dtype, dcnv4_plan* plan);

/*
 * The kernels dcnv4_backward would launch for these arguments (for reporting
 * and tests).  Pure host computation, no HIP call.  need_x / need_offset_or_mask
 * say which gradient pointers would be non-NULL.
 */
typedef struct dcnv4_backward_plan {
    int x_path;        /* 0 no grad_x; 1 LDS fixed point over the whole bordered
                          image; 2 LDS fixed point in square tiles (global atomic
                          adds beyond the margin); 3 global atomic adds */
    int x_channels;    /* paths 1, 2: channels per workgroup */
    int x_tile;        /* path 2: tile side in pixels */
    int x_margin;      /* path 2: pixels around a tile whose units it visits */
    int x_lds_bytes;   /* paths 1, 2: LDS per workgroup, static included */
    int om_path;       /* 0 none; 1 corners from LDS windows; 2 global gathers */
    int om_tile_h, om_tile_w; /* om_path 1: output tile per workgroup */
    int om_lds_bytes;  /* om_path 1: LDS per workgroup */
} dcnv4_backward_plan;

int dcnv4_query_backward_plan(const void* x, const void* offset, const void* mask, const void* grad_out,
                              int need_x, int need_offset_or_mask,
                              int N, int H, int W, int G, int Cg,
                              int K, int stride, int pad, int dilation, float offset_scale,
                              int remove_center, int64_t offset_row, int64_t mask_row,
                              int dtype, dcnv4_backward_plan* plan);

/* Name of a kernel family id from dcnv4_plan (static text). */
const char* dcnv4_kernel_name(int kernel);

#ifdef __cplusplus
}
#endif

#endif /* DCNV4_H */

// DCNv4 forward: the C ABI (include/dcnv4.h) -- validation, planning, launch.
//
// Every argument is checked on the host before the first HIP call, so an
// invalid call launches nothing and writes nothing.  The only global state is
// a per-device cache of "is this a gfx950 device" and its compute-unit count,
// filled on first use.

#include <math.h>
#include <stdarg.h>
#include <stdlib.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "dcnv4.h"
#include "dcnv4_internal.h"

namespace {
thread_local char g_last_error[256] = "";
}  // namespace

namespace dcnv4 {

int fail(int status, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

void clear_error() { g_last_error[0] = '\0'; }

}  // namespace dcnv4

namespace {

using dcnv4::fail;

int out_dim(int in, int K, int stride, int pad, int dil)
{
    if (in < 1 || K < 1 || stride < 1 || pad < 0 || dil < 1) return 0;
    const int64_t span = (int64_t)in + 2 * (int64_t)pad - (int64_t)dil * (K - 1) - 1;
    if (span < 0) return 0;
    const int64_t o = span / stride + 1;
    return o > INT32_MAX ? 0 : (int)o;
}

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

using dcnv4::planner_cus;

// Validate and fill a Problem.  Returns DCNV4_OK or an error status.  With
// check_pointers false only the shapes and parameters are checked (the
// backward checks its own pointers).
int validate(dcnv4::Problem* p, const void* x, const void* offset, const void* mask,
             const void* out, int N, int H, int W, int G, int Cg, int K, int stride,
             int pad, int dil, float offset_scale, int remove_center,
             int64_t offset_row, int64_t mask_row, int dtype, bool check_pointers = true)
{
    g_last_error[0] = '\0';
    if (dtype != DCNV4_F32 && dtype != DCNV4_F16 && dtype != DCNV4_BF16)
        return fail(DCNV4_ERR_DTYPE, "dtype %d is not f32 (0), f16 (1) or bf16 (2)", dtype);
    if (N < 0 || H < 1 || W < 1 || G < 1 || Cg < 1)
        return fail(DCNV4_ERR_SHAPE, "need N >= 0 and H, W, G, Cg >= 1 (got N=%d H=%d W=%d G=%d Cg=%d)",
                    N, H, W, G, Cg);
    if (K < 1 || stride < 1 || dil < 1 || pad < 0)
        return fail(DCNV4_ERR_PARAM, "need K, stride, dilation >= 1 and pad >= 0 (got K=%d s=%d d=%d p=%d)",
                    K, stride, dil, pad);
    if (!isfinite(offset_scale))
        return fail(DCNV4_ERR_PARAM, "offset_scale is not finite");
    if (remove_center != 0 && remove_center != 1)
        return fail(DCNV4_ERR_PARAM, "remove_center must be 0 or 1");
    if (remove_center && (K % 2 == 0 || K < 3))
        return fail(DCNV4_ERR_PARAM, "remove_center needs an odd K >= 3 (got K=%d)", K);
    if (H >= (1 << 24) || W >= (1 << 24))
        return fail(DCNV4_ERR_TOO_LARGE, "H and W must be < 2^24 (positions are exact in binary32)");
    if ((int64_t)K * K > 1024)
        return fail(DCNV4_ERR_PARAM, "K*K must be <= 1024");
    const int Ho = out_dim(H, K, stride, pad, dil), Wo = out_dim(W, K, stride, pad, dil);
    if (Ho < 1 || Wo < 1)
        return fail(DCNV4_ERR_PARAM, "no output: Ho=%d Wo=%d", Ho, Wo);
    const int P = K * K - remove_center;
    const int64_t C = (int64_t)G * Cg;
    if (C >= ((int64_t)1 << 31))
        return fail(DCNV4_ERR_TOO_LARGE, "G*Cg must be < 2^31");
    const int64_t dense_off = (int64_t)G * 2 * P, dense_mask = (int64_t)G * P;
    if (offset_row == 0) offset_row = dense_off;
    if (mask_row == 0) mask_row = dense_mask;
    if (offset_row < dense_off || mask_row < dense_mask)
        return fail(DCNV4_ERR_PARAM, "row strides must be >= G*2*P (%lld) and G*P (%lld)",
                    (long long)dense_off, (long long)dense_mask);
    {
        // one image of each tensor must span < 2^31 bytes (32-bit buffer offsets)
        const int64_t s = dtype == DCNV4_F32 ? 4 : 2, lim = (int64_t)1 << 31;
        const int64_t hw = (int64_t)Ho * Wo;
        if ((int64_t)H * W * C * s >= lim || hw * C * s >= lim ||
            ((hw - 1) * offset_row + dense_off) * s >= lim || ((hw - 1) * mask_row + dense_mask) * s >= lim)
            return fail(DCNV4_ERR_TOO_LARGE, "one image of x, out, offset or mask must span < 2^31 bytes");
    }
    const int64_t units = (int64_t)N * Ho * Wo * G;
    if (units >= ((int64_t)1 << 31))
        return fail(DCNV4_ERR_TOO_LARGE, "N*Ho*Wo*G must be < 2^31");

    p->x = x; p->off = offset; p->msk = mask; p->out = (void*)out;
    p->N = N; p->H = H; p->W = W; p->G = G; p->Cg = Cg; p->K = K; p->P = P;
    p->stride = stride; p->pad = pad; p->dil = dil; p->Ho = Ho; p->Wo = Wo;
    p->remove_center = remove_center; p->softmax = 0; p->off_row = offset_row; p->mask_row = mask_row;
    p->offset_scale = offset_scale; p->dtype = dtype;
    p->cus = planner_cus(0);
    if (N == 0 || !check_pointers) return DCNV4_OK;

    if (!x || !offset || !mask || !out)
        return fail(DCNV4_ERR_NULL, "null pointer (x=%p offset=%p mask=%p out=%p)", x, offset, mask, out);
    const int s = dtype == DCNV4_F32 ? 4 : 2;
    if ((uintptr_t)x % s || (uintptr_t)offset % s || (uintptr_t)mask % s || (uintptr_t)out % s)
        return fail(DCNV4_ERR_ALIGN, "pointers must be aligned to the %d-byte element size", s);
    const int64_t npix_out = (int64_t)N * Ho * Wo;
    const int64_t xbytes = (int64_t)N * H * W * C * s;
    const int64_t obytes = npix_out * C * s;
    const int64_t offbytes = ((npix_out - 1) * offset_row + dense_off) * s;
    const int64_t mbytes = ((npix_out - 1) * mask_row + dense_mask) * s;
    if (overlaps(out, obytes, x, xbytes) || overlaps(out, obytes, offset, offbytes) ||
        overlaps(out, obytes, mask, mbytes))
        return fail(DCNV4_ERR_ALIAS, "out overlaps an input");
    return DCNV4_OK;
}

}  // namespace

namespace dcnv4 {

// Compute units the planners size their grids for: DCNV4_CUS (1..4096) when
// set (tests of the planners; a partitioned device), else the device's count,
// else (plan queries, which make no HIP call) an MI355X's 256.
int planner_cus(int device_cus)
{
    if (const char* e = getenv("DCNV4_CUS")) {
        const int v = atoi(e);
        if (v >= 1 && v <= 4096) return v;
    }
    return device_cus > 0 ? device_cus : kDefaultCus;
}

// Is the current device a gfx950?  Cached per device id, with its compute
// unit count (multiProcessorCount), returned in *cus.
int check_device(int* cus)
{
    static std::mutex mu;
    static int cache[64];   // 0 unknown, 1 yes, 2 no
    static int cu_count[64];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(DCNV4_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64)
        return fail(DCNV4_ERR_HIP, "device id %d out of range", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess)
            return fail(DCNV4_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
        cache[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        cu_count[dev] = prop.multiProcessorCount;
        if (cache[dev] == 2)
            return fail(DCNV4_ERR_HIP, "device %d is %s; this library is built for gfx950", dev,
                        prop.gcnArchName);
    }
    if (cache[dev] != 1)
        return fail(DCNV4_ERR_HIP, "device %d is not a gfx950", dev);
    *cus = cu_count[dev];
    return DCNV4_OK;
}

}  // namespace dcnv4

namespace {

using dcnv4::check_device;

int forward_impl(const void* x, const void* offset, const void* mask, void* out,
                 int N, int H, int W, int G, int Cg, int K, int stride, int pad, int dil,
                 float offset_scale, int remove_center, int64_t offset_row, int64_t mask_row,
                 int dtype, void* stream, int softmax = 0)
{
    dcnv4::Problem p;
    int st = validate(&p, x, offset, mask, out, N, H, W, G, Cg, K, stride, pad, dil,
                      offset_scale, remove_center, offset_row, mask_row, dtype);
    p.softmax = softmax;
    if (st != DCNV4_OK || N == 0) return st;
    int cus = 0;
    st = check_device(&cus);
    if (st != DCNV4_OK) return st;
    p.cus = planner_cus(cus);
    dcnv4::Plan plan;
    dcnv4::make_plan(p, &plan);
    const hipError_t e = dcnv4::launch_forward(p, plan, (hipStream_t)stream);
    if (e != hipSuccess)
        return fail(DCNV4_ERR_HIP, "launch of %s failed: %s", dcnv4_kernel_name(plan.kernel),
                    hipGetErrorString(e));
    return DCNV4_OK;
}

int backward_impl(const void* x, const void* offset, const void* mask, const void* grad_out,
                  float* grad_x, float* grad_offset, float* grad_mask,
                  int N, int H, int W, int G, int Cg, int K, int stride, int pad, int dil,
                  float offset_scale, int remove_center, int64_t offset_row, int64_t mask_row,
                  int dtype, void* stream)
{
    dcnv4::Problem p;
    int st = validate(&p, x, offset, mask, nullptr, N, H, W, G, Cg, K, stride, pad, dil,
                      offset_scale, remove_center, offset_row, mask_row, dtype, false);
    if (st != DCNV4_OK) return st;
    {
        // binary32 gradients: one image of grad_x, grad_offset, grad_mask < 2^31 bytes
        const int64_t lim = (int64_t)1 << 31, hw = (int64_t)p.Ho * p.Wo;
        const int64_t C = (int64_t)G * Cg;
        if ((int64_t)H * W * C * 4 >= lim || ((hw - 1) * p.off_row + (int64_t)G * 2 * p.P) * 4 >= lim ||
            ((hw - 1) * p.mask_row + (int64_t)G * p.P) * 4 >= lim)
            return fail(DCNV4_ERR_TOO_LARGE, "one image of a binary32 gradient must span < 2^31 bytes");
    }
    if (N == 0) return DCNV4_OK;
    if (!x || !offset || !mask || !grad_out)
        return fail(DCNV4_ERR_NULL, "null input pointer (x=%p offset=%p mask=%p grad_out=%p)", x, offset, mask,
                    grad_out);
    const int s = dtype == DCNV4_F32 ? 4 : 2;
    if ((uintptr_t)x % s || (uintptr_t)offset % s || (uintptr_t)mask % s || (uintptr_t)grad_out % s ||
        (uintptr_t)grad_x % 4 || (uintptr_t)grad_offset % 4 || (uintptr_t)grad_mask % 4)
        return fail(DCNV4_ERR_ALIGN, "inputs must be aligned to %d bytes and gradients to 4", s);
    if (dcnv4::backward_vec_bytes(p, grad_out) * 64 < Cg * s)
        return fail(DCNV4_ERR_TOO_LARGE, "the backward handles up to 64 vectors per group: Cg*s = %d bytes is too many "
                    "for this alignment", Cg * s);
    const int64_t C = (int64_t)G * Cg, npix = (int64_t)N * p.Ho * p.Wo;
    const int64_t xb = (int64_t)N * H * W * C * s, ob = npix * C * s;
    const int64_t offb = ((npix - 1) * p.off_row + (int64_t)G * 2 * p.P) * s;
    const int64_t mb = ((npix - 1) * p.mask_row + (int64_t)G * p.P) * s;
    const int64_t gxb = (int64_t)N * H * W * C * 4;
    const int64_t goffb = ((npix - 1) * p.off_row + (int64_t)G * 2 * p.P) * 4;
    const int64_t gmb = ((npix - 1) * p.mask_row + (int64_t)G * p.P) * 4;
    struct Span { const void* p; int64_t b; };
    const Span in[4] = {{x, xb}, {offset, offb}, {mask, mb}, {grad_out, ob}};
    const Span outs[3] = {{grad_x, gxb}, {grad_offset, goffb}, {grad_mask, gmb}};
    for (const Span& o : outs) {
        if (!o.p) continue;
        for (const Span& i : in)
            if (overlaps(o.p, o.b, i.p, i.b)) return fail(DCNV4_ERR_ALIAS, "a gradient overlaps an input");
    }
    if (grad_x && ((grad_offset && overlaps(grad_x, gxb, grad_offset, goffb)) ||
                   (grad_mask && overlaps(grad_x, gxb, grad_mask, gmb))))
        return fail(DCNV4_ERR_ALIAS, "grad_x overlaps grad_offset or grad_mask");
    if (!grad_x && !grad_offset && !grad_mask) return DCNV4_OK;
    int cus = 0;
    st = check_device(&cus);
    if (st != DCNV4_OK) return st;
    p.cus = planner_cus(cus);
    const hipError_t e = dcnv4::launch_backward(p, grad_out, grad_x, grad_offset, grad_mask, (hipStream_t)stream);
    if (e != hipSuccess) return fail(DCNV4_ERR_HIP, "launch of the backward failed: %s", hipGetErrorString(e));
    return DCNV4_OK;
}

}  // namespace

extern "C" {

int dcnv4_backward(const void* x, const void* offset, const void* mask, const void* grad_out,
                   float* grad_x, float* grad_offset, float* grad_mask,
                   int N, int H, int W, int G, int Cg,
                   int K, int stride, int pad, int dilation, float offset_scale,
                   int remove_center, int64_t offset_row, int64_t mask_row,
                   int dtype, void* stream)
{
    return backward_impl(x, offset, mask, grad_out, grad_x, grad_offset, grad_mask, N, H, W, G, Cg, K, stride,
                         pad, dilation, offset_scale, remove_center, offset_row, mask_row, dtype, stream);
}

int dcnv4_forward(const void* x, const void* offset, const void* mask, void* out,
                  int N, int H, int W, int G, int Cg,
                  int K, int stride, int pad, int dilation, float offset_scale,
                  int dtype, void* stream)
{
    return forward_impl(x, offset, mask, out, N, H, W, G, Cg, K, stride, pad, dilation,
                        offset_scale, 0, 0, 0, dtype, stream);
}

int dcnv4_forward_ex(const void* x, const void* offset, const void* mask, void* out,
                     int N, int H, int W, int G, int Cg,
                     int K, int stride, int pad, int dilation, float offset_scale,
                     int remove_center, int64_t offset_row, int64_t mask_row,
                     int dtype, void* stream)
{
    return forward_impl(x, offset, mask, out, N, H, W, G, Cg, K, stride, pad, dilation,
                        offset_scale, remove_center, offset_row, mask_row, dtype, stream);
}

int dcnv4_forward_softmax(const void* x, const void* offset, const void* mask, void* out,
                          int N, int H, int W, int G, int Cg,
                          int K, int stride, int pad, int dilation, float offset_scale,
                          int remove_center, int64_t offset_row, int64_t mask_row,
                          int dtype, void* stream)
{
    return forward_impl(x, offset, mask, out, N, H, W, G, Cg, K, stride, pad, dilation,
                        offset_scale, remove_center, offset_row, mask_row, dtype, stream, 1);
}

int dcnv4_output_dim(int in, int K, int stride, int pad, int dilation)
{
    return out_dim(in, K, stride, pad, dilation);
}

const char* dcnv4_status_string(int status)
{
    switch (status) {
        case DCNV4_OK: return "ok";
        case DCNV4_ERR_NULL: return "null pointer";
        case DCNV4_ERR_SHAPE: return "invalid shape";
        case DCNV4_ERR_PARAM: return "invalid parameter";
        case DCNV4_ERR_DTYPE: return "invalid dtype";
        case DCNV4_ERR_ALIAS: return "output overlaps an input";
        case DCNV4_ERR_TOO_LARGE: return "problem too large";
        case DCNV4_ERR_HIP: return "HIP error";
        case DCNV4_ERR_ALIGN: return "misaligned pointer";
        default: return "unknown status";
    }
}

const char* dcnv4_last_error(void) { return g_last_error; }

const char* dcnv4_version(void) { return "0.1.0"; }

int dcnv4_query_plan(const void* x, const void* offset, const void* mask, const void* out,
                     int N, int H, int W, int G, int Cg,
                     int K, int stride, int pad, int dilation, float offset_scale,
                     int remove_center, int64_t offset_row, int64_t mask_row,
                     int dtype, dcnv4_plan* plan)
{
    if (!plan) return fail(DCNV4_ERR_NULL, "plan is null");
    dcnv4::Problem p;
    const int st = validate(&p, x, offset, mask, out, N, H, W, G, Cg, K, stride, pad, dilation,
                            offset_scale, remove_center, offset_row, mask_row, dtype);
    if (st != DCNV4_OK) return st;
    dcnv4::Plan pl;
    dcnv4::make_plan(p, &pl);
    memset(plan, 0, sizeof *plan);
    plan->kernel = pl.kernel;
    plan->vec = pl.vec;
    plan->lanes_per_unit = pl.lanes;
    plan->block = pl.block;
    plan->grid = N == 0 ? 0 : pl.grid;
    plan->groups_per_block = pl.GB;
    plan->tile_h = pl.TH;
    plan->tile_w = pl.TW;
    plan->margin_y = pl.RY;
    plan->margin_x = pl.RX;
    plan->window_h = pl.WH;
    plan->window_w = pl.WW;
    plan->full_window = pl.full;
    plan->lds_bytes = pl.lds_total;
    plan->coalesced_offsets = pl.coal;
    plan->shared_coefficients = pl.kernel == dcnv4::kKernelWindow ? pl.share : 0;
    return DCNV4_OK;
}

int dcnv4_query_backward_plan(const void* x, const void* offset, const void* mask, const void* grad_out,
                              int need_x, int need_offset_or_mask,
                              int N, int H, int W, int G, int Cg,
                              int K, int stride, int pad, int dilation, float offset_scale,
                              int remove_center, int64_t offset_row, int64_t mask_row,
                              int dtype, dcnv4_backward_plan* plan)
{
    if (!plan) return fail(DCNV4_ERR_NULL, "plan is null");
    dcnv4::Problem p;
    const int st = validate(&p, x, offset, mask, nullptr, N, H, W, G, Cg, K, stride, pad, dilation,
                            offset_scale, remove_center, offset_row, mask_row, dtype, false);
    if (st != DCNV4_OK) return st;
    dcnv4::BwdPlan bp;
    dcnv4::plan_backward(p, grad_out, need_x != 0, need_offset_or_mask != 0, &bp);
    memset(plan, 0, sizeof *plan);
    plan->x_path = bp.x_path;
    plan->x_channels = bp.cc;
    plan->x_tile = bp.x_path == 2 ? 1 << bp.tile_sh : 0;
    plan->x_margin = bp.x_path == 2 ? bp.margin : 0;
    plan->x_lds_bytes = bp.x_lds;
    plan->om_path = bp.om_path;
    if (bp.om_path == 1) {
        plan->om_tile_h = bp.om.th;
        plan->om_tile_w = bp.om.tw;
        plan->om_lds_bytes = (int)bp.om.lds;
    }
    return DCNV4_OK;
}

const char* dcnv4_kernel_name(int kernel)
{
    switch (kernel) {
        case dcnv4::kKernelDirect: return "direct";
        case dcnv4::kKernelWindow: return "window";
        default: return "none";
    }
}

}  // extern "C"

// DCNv4 module forward: the C ABI of include/dcnv4_module.h -- validation,
// workspace layout, launch.  Every argument is checked before the first HIP
// call; an invalid call launches nothing and writes nothing.

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "dcnv4.h"
#include "dcnv4_internal.h"
#include "dcnv4_module.h"
#include "dcnv4_module_internal.h"

namespace {

using dcnv4::fail;
using dcnv4::ModuleLayout;
using dcnv4::ModuleProblem;

constexpr int kMaxChannels = 4096;

int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return abytes > 0 && bbytes > 0 && a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

// Shapes and options (no pointers); fills the layout.
int validate_config(int N, int H, int W, const dcnv4_module_config* cfg, int dtype, ModuleLayout* L)
{
    dcnv4::clear_error();
    if (!cfg) return fail(DCNV4_ERR_NULL, "config is null");
    if (dtype != DCNV4_F32 && dtype != DCNV4_F16 && dtype != DCNV4_BF16)
        return fail(DCNV4_ERR_DTYPE, "dtype %d is not f32 (0), f16 (1) or bf16 (2)", dtype);
    const int Cin = cfg->Cin, G = cfg->G, Cg = cfg->Cg;
    if (N < 0 || H < 1 || W < 1 || Cin < 1 || G < 1 || Cg < 1)
        return fail(DCNV4_ERR_SHAPE, "need N >= 0 and H, W, Cin, G, Cg >= 1");
    const int64_t C = (int64_t)G * Cg;
    if (C > kMaxChannels || Cin > kMaxChannels)
        return fail(DCNV4_ERR_TOO_LARGE, "Cin and G*Cg must be at most %d", kMaxChannels);
    if (cfg->out_proj != 0 && cfg->out_proj != 1) return fail(DCNV4_ERR_PARAM, "out_proj must be 0 or 1");
    if (cfg->out_proj && (cfg->Cout < 1 || cfg->Cout > kMaxChannels))
        return fail(DCNV4_ERR_SHAPE, "Cout must be in 1..%d", kMaxChannels);
    if (!cfg->out_proj && cfg->Cout != (int)C)
        return fail(DCNV4_ERR_SHAPE, "without the output projection Cout must equal G*Cg (%lld)", (long long)C);
    const int s = dtype == DCNV4_F32 ? 4 : 2;
    if (s == 2 && (Cin % 4 || C % 4))
        return fail(DCNV4_ERR_SHAPE, "16-bit types need Cin and G*Cg to be multiples of 4 (matrix-core loads)");
    if (cfg->norm != DCNV4_NORM_NONE && cfg->norm != DCNV4_NORM_GROUP && cfg->norm != DCNV4_NORM_LAYER)
        return fail(DCNV4_ERR_PARAM, "norm must be 0 (none), 1 (group) or 2 (layer)");
    if (cfg->norm == DCNV4_NORM_GROUP && (cfg->norm_groups < 1 || C % cfg->norm_groups))
        return fail(DCNV4_ERR_PARAM, "norm_groups must divide G*Cg");
    if (cfg->norm != DCNV4_NORM_NONE && !(cfg->eps > 0.0f && isfinite(cfg->eps)))
        return fail(DCNV4_ERR_PARAM, "eps must be finite and > 0");
    if ((cfg->remove_center != 0 && cfg->remove_center != 1) || (cfg->center_scale != 0 && cfg->center_scale != 1))
        return fail(DCNV4_ERR_PARAM, "remove_center and center_scale must be 0 or 1");
    if (!isfinite(cfg->offset_scale)) return fail(DCNV4_ERR_PARAM, "offset_scale is not finite");
    if (H >= (1 << 24) || W >= (1 << 24)) return fail(DCNV4_ERR_TOO_LARGE, "H and W must be < 2^24");
    const int P = 9 - cfg->remove_center;
    const int R = 3 * G * P + (cfg->center_scale ? G : 0);
    const int64_t rs = (R + 7) / 8 * 8;
    const int64_t hw = (int64_t)H * W, lim = (int64_t)1 << 31;
    if (hw * C * s >= lim || hw * rs * s >= lim || hw * Cin * s >= lim ||
        (cfg->out_proj && hw * cfg->Cout * s >= lim))
        return fail(DCNV4_ERR_TOO_LARGE, "one image of a tensor must span < 2^31 bytes");
    const int64_t M = (int64_t)N * hw;
    if (M * G >= lim || M >= lim / 4) return fail(DCNV4_ERR_TOO_LARGE, "N*H*W*G must be < 2^31");
    L->P = P;
    L->R = R;
    L->rows_stride = rs;
    // group-norm partial sums: enough (image, slice) blocks to fill the GPU,
    // slices of at least 64 pixels
    int slices = (int)((1024 + (N > 0 ? N : 1) - 1) / (N > 0 ? N : 1));
    const int maxs = (int)(hw / 64 > 0 ? hw / 64 : 1);
    slices = slices < 1 ? 1 : slices > maxs ? maxs : slices;
    L->slices = slices;
    int64_t at = 0;
    auto region = [&](bool used, int64_t bytes) {
        if (!used) return (int64_t)-1;
        const int64_t r = at;
        at = align256(at + bytes);
        return r;
    };
    const int64_t act = M * C * s;
    L->xp = region(true, act);
    L->xn = region(cfg->norm != DCNV4_NORM_NONE, act);
    L->d = region(true, act);
    L->rows = region(true, M * rs * s);
    L->y = region(cfg->center_scale || cfg->out_proj, act);
    L->gated = region(cfg->center_scale && cfg->out_proj, act);
    const int64_t part = (int64_t)N * slices * C * 2 * 8;
    L->stat_offset = align256(part);
    L->stats = region(cfg->norm == DCNV4_NORM_GROUP, L->stat_offset + (int64_t)N * cfg->norm_groups * 2 * 4);
    L->total = at;
    return DCNV4_OK;
}

}  // namespace

extern "C" {

int dcnv4_module_workspace_layout(int N, int H, int W, const dcnv4_module_config* cfg, int dtype,
                                  dcnv4_module_layout* layout)
{
    if (!layout) return fail(DCNV4_ERR_NULL, "layout is null");
    ModuleLayout L;
    const int st = validate_config(N, H, W, cfg, dtype, &L);
    if (st != DCNV4_OK) return st;
    layout->xp = L.xp;
    layout->xn = L.xn;
    layout->d = L.d;
    layout->rows = L.rows;
    layout->y = L.y;
    layout->gated = L.gated;
    layout->stats = L.stats;
    layout->rows_stride = L.rows_stride;
    layout->total = L.total;
    return DCNV4_OK;
}

}  // extern "C"

namespace {

// Validate a call whose workspace is `workspace` (workspace_bytes) and launch it.
int module_forward_impl(const void* x_in, const dcnv4_module_weights* w, void* out, int N, int H, int W,
                        const dcnv4_module_config* cfg, void* workspace, size_t workspace_bytes, int dtype,
                        void* stream, const ModuleLayout& L)
{
    int st;
    if (N == 0) return DCNV4_OK;
    if (!w) return fail(DCNV4_ERR_NULL, "weights is null");
    const bool gn = cfg->norm != DCNV4_NORM_NONE;
    if (!x_in || !out || !workspace || !w->w_in || !w->b_in || !w->w_dw || !w->b_dw || !w->w_pred ||
        !w->b_pred || (gn && (!w->gamma || !w->beta)) || (cfg->out_proj && (!w->w_out || !w->b_out)))
        return fail(DCNV4_ERR_NULL, "a tensor or weight pointer the configuration needs is null");
    const int s = dtype == DCNV4_F32 ? 4 : 2;
    if ((uintptr_t)workspace % 256) return fail(DCNV4_ERR_ALIGN, "workspace must be 256-byte aligned");
    if ((uintptr_t)x_in % s || (uintptr_t)out % s || (uintptr_t)w->w_in % s || (uintptr_t)w->w_pred % s ||
        (cfg->out_proj && (uintptr_t)w->w_out % s))
        return fail(DCNV4_ERR_ALIGN, "tensors must be aligned to the element size");
    if (s == 2 && ((uintptr_t)x_in % 8 || (uintptr_t)w->w_in % 8 || (uintptr_t)w->w_pred % 8 ||
                   (cfg->out_proj && (uintptr_t)w->w_out % 8)))
        return fail(DCNV4_ERR_ALIGN, "16-bit matrices and x_in must be 8-byte aligned (matrix-core loads)");
    if ((int64_t)workspace_bytes < L.total)
        return fail(DCNV4_ERR_TOO_LARGE, "workspace of %zu bytes, %lld needed", workspace_bytes, (long long)L.total);
    const int64_t C = (int64_t)cfg->G * cfg->Cg, M = (int64_t)N * H * W;
    const int64_t xb = M * cfg->Cin * s, ob = M * cfg->Cout * s, wsb = (int64_t)workspace_bytes;
    if (overlaps(out, ob, x_in, xb) || overlaps(out, ob, workspace, wsb) || overlaps(workspace, wsb, x_in, xb))
        return fail(DCNV4_ERR_ALIAS, "out, x_in and the workspace must not overlap");
    struct Span { const void* p; int64_t b; };
    const Span ws[] = {{w->w_in, C * cfg->Cin * s}, {w->b_in, C * 4}, {w->gamma, gn ? C * 4 : 0},
                       {w->beta, gn ? C * 4 : 0}, {w->w_dw, C * 9 * 4}, {w->b_dw, C * 4},
                       {w->w_pred, (int64_t)L.R * C * s}, {w->b_pred, (int64_t)L.R * 4},
                       {w->w_out, cfg->out_proj ? (int64_t)cfg->Cout * C * s : 0},
                       {w->b_out, cfg->out_proj ? (int64_t)cfg->Cout * 4 : 0}};
    for (const Span& sp : ws)
        if (sp.p && (overlaps(sp.p, sp.b, workspace, wsb) || overlaps(sp.p, sp.b, out, ob)))
            return fail(DCNV4_ERR_ALIAS, "a weight overlaps the workspace or out");
    int cus = 0;
    st = dcnv4::check_device(&cus);
    if (st != DCNV4_OK) return st;
    ModuleProblem m;
    memset(&m, 0, sizeof m);
    m.x_in = x_in;
    m.w = *w;
    m.out = out;
    m.workspace = workspace;
    m.N = N; m.H = H; m.W = W; m.Cin = cfg->Cin; m.G = cfg->G; m.Cg = cfg->Cg; m.Cout = cfg->Cout;
    m.norm = cfg->norm; m.norm_groups = cfg->norm == DCNV4_NORM_GROUP ? cfg->norm_groups : 1;
    m.eps = cfg->eps;
    m.remove_center = cfg->remove_center; m.center_scale = cfg->center_scale; m.out_proj = cfg->out_proj;
    m.offset_scale = cfg->offset_scale;
    m.dtype = dtype;
    m.cus = dcnv4::planner_cus(cus);
    m.layout = L;
    const hipError_t e = dcnv4::launch_module(m, (hipStream_t)stream);
    if (e != hipSuccess) return fail(DCNV4_ERR_HIP, "launch of the module failed: %s", hipGetErrorString(e));
    return DCNV4_OK;
}


// The no-allocation variant's workspace: one array per device, in the code
// object's data (loaded with the library), never allocated or freed by a
// call.  Host code uses only its device address from hipGetSymbolAddress:
// the array's name stands for a host-side shadow, not device memory.
static __device__ __align__(256) unsigned char scratch[DCNV4_MODULE_SCRATCH_BYTES];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr after a failure
// (recorded as the call's error).
void* scratch_address()
{
    static std::mutex mu;
    static void* addr[64];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        fail(DCNV4_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
        return nullptr;
    }
    if (dev < 0 || dev >= 64) {
        fail(DCNV4_ERR_HIP, "device id %d out of range", dev);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            fail(DCNV4_ERR_HIP, "hipGetSymbolAddress of the module scratch array: %s", hipGetErrorString(e));
            return nullptr;
        }
        addr[dev] = p;
    }
    return addr[dev];
}

}  // namespace

extern "C" {

int dcnv4_module_forward(const void* x_in, const dcnv4_module_weights* w, void* out,
                         int N, int H, int W, const dcnv4_module_config* cfg,
                         void* workspace, size_t workspace_bytes, int dtype, void* stream)
{
    ModuleLayout L;
    const int st = validate_config(N, H, W, cfg, dtype, &L);
    if (st != DCNV4_OK) return st;
    return module_forward_impl(x_in, w, out, N, H, W, cfg, workspace, workspace_bytes, dtype, stream, L);
}

int dcnv4_module_forward_noalloc(const void* x_in, const dcnv4_module_weights* w, void* out,
                                 int N, int H, int W, const dcnv4_module_config* cfg, int dtype, void* stream)
{
    ModuleLayout L;
    const int st = validate_config(N, H, W, cfg, dtype, &L);
    if (st != DCNV4_OK) return st;
    if (L.total > (int64_t)DCNV4_MODULE_SCRATCH_BYTES)
        return fail(DCNV4_ERR_TOO_LARGE, "the problem needs a %lld-byte workspace; the no-allocation variant holds "
                    "%lld bytes (use dcnv4_module_forward with a workspace)", (long long)L.total,
                    (long long)DCNV4_MODULE_SCRATCH_BYTES);
    if (N == 0) return DCNV4_OK;
    int cus = 0;
    const int dst = dcnv4::check_device(&cus);
    if (dst != DCNV4_OK) return dst;
    void* ws = scratch_address();
    if (!ws) return DCNV4_ERR_HIP;
    return module_forward_impl(x_in, w, out, N, H, W, cfg, ws, (size_t)DCNV4_MODULE_SCRATCH_BYTES, dtype, stream,
                               L);
}

}  // extern "C"

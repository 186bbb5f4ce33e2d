// Internal interface between the ABI layer (dcnv4_host.hip) and the launch
// planner (dcnv4_launch.hip).  Not installed; the public ABI is include/dcnv4.h.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace dcnv4 {

// One validated forward problem.  Strides and counts in elements of the I/O type.
struct Problem {
    const void* x;
    const void* off;
    const void* msk;
    void* out;
    int N, H, W, G, Cg, K, P, stride, pad, dil, Ho, Wo;
    int remove_center;
    int softmax;            // DCNv3-style: softmax over each group's P weights first
    int64_t off_row, mask_row;
    float offset_scale;
    int dtype;
    int cus;                // compute units the planners size grids for
};

enum KernelId {
    kKernelNone = 0,
    kKernelDirect = 1,   // corner reads from global memory (general path)
    kKernelWindow = 2,   // corner reads from an LDS window of x
};

struct Plan {
    int kernel;
    int vec;        // direct: bytes per lane per corner read
    int lanes;      // lanes per (pixel, group) unit
    int block;      // threads per workgroup
    int64_t grid;   // workgroups (before the XCD round-up of the window family)
    int nv;         // window: 16-byte vectors per unit
    int GB, TH, TW, RY, RX, WH, WW, full;
    int coal;       // window: offset rows staged through LDS per wave
    int lds_bytes;  // dynamic LDS (window)
    int lds_total;  // all LDS per workgroup (the coalesced variant adds static buffers)
    int lpu;        // window: lanes per unit (> 1: one 16-byte vector per lane)
    int share;      // window: split units share their points' coefficients (2 or 4 lanes)
};

// Largest LDS allocation one workgroup may use on gfx950 (the CU's 160 KiB).
constexpr int kLdsPerCu = 160 * 1024;
// Compute units of an MI355X, the planners' count when the device's is not
// known (plan queries make no HIP call).
constexpr int kDefaultCus = 256;
// Static LDS of the x-gradient LDS kernels (per-wave maxima and non-finite
// flags of a 1024-thread workgroup, rounded up): a workgroup's dynamic
// accumulator plane plus this must fit in kLdsPerCu.
constexpr int kBwdXStaticLds = 256;

// The ABI layer's shared pieces (dcnv4_host.hip): record the calling
// thread's last error (returns `status`), clear it, the compute units the
// planners use, and the gfx950 check of the current device (its CU count).
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
int planner_cus(int device_cus);
int check_device(int* cus);

// Pure host: pick the kernel and launch shape for a validated problem.
void make_plan(const Problem& p, Plan* plan);

// Enqueue the kernel chosen by make_plan on `stream`.
hipError_t launch_forward(const Problem& p, const Plan& plan, hipStream_t stream);

// Backward: bytes per lane per vector for these pointers (lanes per unit =
// Cg*s / that), and the launch (zero grad_x, then the gradient kernel).
// Null gradient pointers are skipped.
int backward_vec_bytes(const Problem& p, const void* gout);
// Channels per workgroup of the LDS x-gradient kernel (0: global atomics instead).
int backward_x_chunk(const Problem& p);
// When the whole image does not fit: the tiled LDS x-gradient kernel's
// channels per workgroup, log2 tile side and margin (false: global atomics).
bool backward_x_tiles(const Problem& p, int* cc, int* tile_sh, int* margin);
// Whether the backward's planners replace whole-image kernels whose grid
// cannot fill the GPU by tiled ones (environment DCNV4_BWD_FILL=0: no).
bool backward_fill_gpu();
// Launch shape of the offset/weight-gradient LDS kernel: output tiles of
// th x tw units (the whole image when its bordered copy fits), windows of
// wh x ww pixels from ry / rx pixels before a tile's grid, rows of `pitch`
// 16-byte entries.
struct OmPlan {
    int block, pitch;
    int th, tw, ry, rx, wh, ww, tiles_y, tiles_x;
    size_t lds;
};
// Whether the offset/weight gradients can read their corners from an LDS
// window of each (image, tile, group) (K = 3, one to five 16-byte vectors per
// unit, 16-byte aligned x and output gradient, a window that fits the LDS),
// and how.
bool backward_om_window_plan(const Problem& p, const void* gout, OmPlan* plan);
// What the backward launches for a problem (pure host).  x_path: 0 no x
// gradient, 1 whole-image LDS kernel, 2 tiled LDS kernel, 3 global atomics;
// om_path: 0 no offset/weight gradients, 1 LDS-window kernel, 2 general kernel.
struct BwdPlan {
    int x_path, cc, tile_sh, margin, x_lds;
    int om_path;
    OmPlan om;
};
void plan_backward(const Problem& p, const void* gout, bool want_x, bool want_om, BwdPlan* plan);
hipError_t launch_backward(const Problem& p, const void* gout, float* gx, float* goff, float* gmask,
                           hipStream_t stream);

}  // namespace dcnv4

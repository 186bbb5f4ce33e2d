// Internal interface between the module's ABI layer (dcnv4_module_host.hip)
// and its kernels (dcnv4_module.hip).  Not installed.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "dcnv4_module.h"

namespace dcnv4 {

// Byte offsets in the workspace (-1: region unused) and the derived sizes.
struct ModuleLayout {
    int64_t xp, xn, d, rows, y, gated, stats;
    int64_t stat_offset;   // within stats: the binary32 (mean, rstd) after the binary64 partial sums
    int64_t rows_stride;   // elements per pixel of rows
    int64_t total;
    int P, R;              // operator points, predictor rows
    int slices;            // group-norm partial sums per image
};

// A validated module problem.
struct ModuleProblem {
    const void* x_in;
    dcnv4_module_weights w;
    void* out;
    void* workspace;
    int N, H, W, Cin, G, Cg, Cout;
    int norm, norm_groups;
    float eps;
    int remove_center, center_scale, out_proj;
    float offset_scale;
    int dtype;
    int cus;
    ModuleLayout layout;
};

// Enqueue the module's kernels on `stream`.
hipError_t launch_module(const ModuleProblem& m, hipStream_t stream);

}  // namespace dcnv4

// Internal interface between the ABI layer (dcnv4_host.hip) and the kernels
// (dcnv4_fwd.hip).  Not installed; the public ABI is include/dcnv4.h.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace dcnv4 {

// One validated forward problem.  Element strides and counts are in elements
// of the I/O type.
struct Problem {
    const void* x;
    const void* off;
    const void* msk;
    void* out;
    int N, H, W, G, Cg, K, P, stride, pad, dil, Ho, Wo;
    int remove_center;
    int64_t off_row, mask_row;
    float offset_scale;
    int dtype;
};

enum KernelId {
    kKernelNone = 0,
    kKernelGatherVec = 1,   // lane per (unit, vector of channels)
};

struct Plan {
    int kernel;
    int vec;        // elements per lane per gather
    int lanes;      // lanes per (pixel, group) unit
    int block;      // threads per block
    int64_t grid;   // blocks
};

// Pure host: pick the kernel and launch shape for a validated problem.
void make_plan(const Problem& p, Plan* plan);

// Enqueue the kernel chosen by make_plan on `stream`.
hipError_t launch_forward(const Problem& p, const Plan& plan, hipStream_t stream);

}  // namespace dcnv4

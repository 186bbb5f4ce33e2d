// Kernel argument blocks and launch entry points (internal).
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace dcnv4 {

// Division by a runtime constant d (1 <= d < 2^31) for numerators < 2^31:
// q = (umulhi(n, mul) + n) >> shift.
struct FastDiv {
    uint32_t d, mul, shift;
};

inline FastDiv make_fastdiv(uint32_t d)
{
    FastDiv f;
    f.d = d;
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    f.shift = l;
    f.mul = (uint32_t)((((1ull << l) - d) << 32) / d + 1);
    if (d == 1) { f.mul = 0; f.shift = 0; }
    return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f)
{
    return (__umulhi(n, f.mul) + n) >> f.shift;
}

// Shared by every kernel family: one validated problem, in elements of the
// I/O type unless named *_bytes.
struct KArgs {
    const void* x;
    const void* off;
    const void* msk;
    void* out;
    int H, W, G, Cg, C, K, P, stride, pad, dil, Ho, Wo;
    int remove_center;
    int softmax;                    // weights normalised by a softmax over each group's points
    int64_t off_row, mask_row;      // elements between output pixels
    uint32_t img_x_bytes;           // one image of x
    uint32_t img_off_bytes;         // one image of offsets (rows of its last pixel included)
    uint32_t img_mask_bytes;
    int64_t img_x_elems, img_out_elems;
    int64_t img_off_elems, img_mask_elems;   // image strides of offset / mask (elements)
    float offset_scale;

    // direct family
    int lanes;                      // lanes per unit
    int vec_bytes;                  // bytes per lane per gather
    uint32_t blocks_per_image;
    uint32_t units_img;             // Ho*Wo*G
    FastDiv div_lanes, div_G, div_Wo;

    // window family
    int GB;                         // groups per workgroup
    int TH, TW;                     // output tile
    int RY, RX;                     // window margin beyond the base footprint
    int WH, WW;                     // window rows / cols held in LDS
    int pitch;                      // LDS row pitch in 16-byte entries (>= WW + 2, multiple of 16)
    int slot_bytes;                 // bytes per window pixel = GB*Cg*s
    int full;                       // window covers [-1,H] x [-1,W]
    int coal;                       // offset rows staged through LDS by each wave (GB == 1,
                                    // full-width tiles, dword-aligned rows)
    uint32_t tiles_x, tiles_y, gtiles;
    FastDiv div_GB, div_TW, div_tiles_x, div_tiles_y, div_gtiles, div_CPS, div_pitch;
    uint32_t win_bytes;             // LDS of the window (the per-wave offset buffers follow)
    uint32_t lds_bytes;             // all dynamic LDS
    int lpu;                        // lanes per unit (> 1: one 16-byte vector per lane)
    int nvt;                        // 16-byte vectors per unit
    int share;                      // split units of 2 or 4 lanes share point coefficients
    FastDiv div_lpu;
};

// Backward kernel arguments (elements of the I/O type unless named *_bytes;
// the gradients are binary32 with the inputs' element strides).
struct BArgs {
    const void* x;
    const void* off;
    const void* msk;
    const void* gout;
    float* gx;
    float* goff;
    float* gmask;
    int H, W, G, Cg, C, K, P, stride, pad, dil, Ho, Wo;
    int remove_center;
    int64_t off_row, mask_row;
    int64_t img_x_elems, img_out_elems, img_off_elems, img_mask_elems;
    uint32_t img_x_bytes, img_out_bytes, img_off_bytes, img_mask_bytes;
    float offset_scale;
    int vec_bytes;                  // bytes per lane per vector
    int lanes;                      // lanes per unit (<= 64)
    int units_per_wave;
    int cc;                         // x-gradient LDS kernel: channels per workgroup (0 = atomics path)
    int cbits;                      // x-gradient LDS kernel: log2 bound of the terms per element
    int pitch;                      // offset/weight-gradient LDS kernel: window row pitch (16-byte entries)
    int tile_sh;                    // tiled x-gradient kernel: log2 of the square tile's side (0 = whole image)
    int tiles_y, tiles_x;           // tiled x-gradient kernel: tiles per image along each axis
    int margin;                     // tiled x-gradient kernel: pixels around a tile whose units it visits
    // offset/weight-gradient LDS kernel: output tiles of om_th x om_tw units
    // (the whole image when it fits), windows of om_wh x om_ww pixels
    // starting om_ry / om_rx pixels before the tile's grid
    int om_th, om_tw, om_ry, om_rx, om_wh, om_ww, om_tiles_y, om_tiles_x;
    FastDiv div_om_tw;
    uint32_t units_img;
    int64_t units_total;
    FastDiv div_units_img, div_G, div_Wo;
};

hipError_t launch_direct(const KArgs& a, int dtype, int block, int64_t grid, hipStream_t stream);
// Offset/weight gradients with a window of each (image, tile, group) in LDS
// (the tile shape in a.om_*): N * tiles * G workgroups of `block` threads,
// `lds` bytes of window, 16-byte vectors per unit nv (1 to 4; 1 to 3 in bf16).
hipError_t launch_backward_om_window(const BArgs& a, int dtype, int nv, int block, size_t lds,
                                     hipStream_t stream);
hipError_t launch_window(const KArgs& a, int dtype, int nv, int block, int64_t grid, hipStream_t stream);
// The same launch with softmax-normalised weights (a.softmax, the DCNv3-style form).
hipError_t launch_window_softmax(const KArgs& a, int dtype, int nv, int block, int64_t grid, hipStream_t stream);

// Window kernel limits the planner needs: threads per workgroup it is
// compiled for, and the LDS of the per-wave offset buffers of its
// coalesced-offset variant for a workgroup of `block` threads.
int window_max_block(int nv);
int window_coal_lds_bytes(int block, int dtype, int P);

}  // namespace dcnv4

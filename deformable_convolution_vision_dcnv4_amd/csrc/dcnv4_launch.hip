// Launch planning for the DCNv4 forward: which kernel family, which tile,
// which workgroup size.  Pure host code apart from the final launch.
//
// Rules (see the kernel files for the why; the choices were measured on the
// FlashInternImage-T stage shapes, the 256x256 dense-prediction shape and the
// 64x64 latent shape):
//   window family when K = 3, Cg*s is a whole number of 16-byte vectors (1..5
//   of them) and x and out are 16-byte aligned, and one of these fits:
//     - the whole zero-bordered image, [-1,H] x [-1,W], for GB groups at
//       once: the smallest GB whose workgroup has at least 128 units, else
//       the largest that fits.  No point can leave such a window, and its
//       workgroups read the fewest bytes per CU; one group per workgroup
//       measured fastest wherever it fits;
//     - else bands of full-width output rows with a margin of R rows for the
//       offsets (R = 5 unless tuned), for the smallest GB, when at most four
//       bands (eight for units of three or more vectors) cover the image:
//       band height chosen to minimise (rounds of workgroups) x (rows
//       computed + rows staged / 2); a margin of R - 1 when that saves a
//       whole round of workgroups.  With more bands the margins cost more
//       staging than LDS saves, and large offsets (whose units fall back to
//       global reads) make it worse;
//     - else tiles of 16 x 64 outputs with a margin of 12 pixels (units of
//       two or more vectors, one lane per vector);
//   a plan with fewer workgroups than CUs (small batches) takes more bands,
//   of at least 7 rows, to fill the GPU, else the direct family: a
//   workgroup holds its CU for its whole tile, so an underfilled grid
//   leaves CUs idle (batch 1 of the stage-1 shape: 31 us on 4 workgroups
//   against 6 us for the direct kernel);
//   units of three or more 16-byte vectors take one lane per vector (measured
//   8-15% faster than whole-unit lanes, which cap a workgroup at 512
//   threads); threads per workgroup: the kernel's maximum, or fewer when one
//   pass covers the tile.  The direct family otherwise.
// DCNV4_TUNE (environment, parsed again whenever its text changes)
// overrides the choices for tuning runs and tests; an explicit kernel, tile
// height or width, group count or full=0|1 turns the GPU-filling rule off:
// "kernel=direct|window,gb=G,th=T,tw=T,r=R,block=B,full=0|1,pitch_add=E,coal=0|1,split=0|1,share=0|1".

#include <stdio.h>
#include <stdlib.h>
#include <string.h>


#include "dcnv4.h"
#include "dcnv4_internal.h"
#include "dcnv4_kernels.h"

namespace dcnv4 {
namespace {

struct Tune {
    int kernel = 0;     // 0 auto, 1 direct, 2 window
    int gb = 0, th = 0, tw = 0, r = -1, block = 0, full = -1, pitch_add = 0, coal = -1, split = -1;
    int share = -1;          // split units of 2 or 4 lanes share point coefficients
};

// Parsed per thread, again whenever the variable's text changes.
const Tune& tune()
{
    thread_local Tune t;
    thread_local char seen[256] = {1, 0};   // never a variable's text: forces the first parse
    const char* env = getenv("DCNV4_TUNE");
    if (!env) env = "";
    if (strncmp(env, seen, sizeof seen) == 0) return t;
    strncpy(seen, env, sizeof seen - 1);
    seen[sizeof seen - 1] = '\0';
    t = Tune();
    {
        char buf[256];
        strncpy(buf, env, sizeof buf - 1);
        buf[sizeof buf - 1] = '\0';
        char* save = nullptr;   // strtok_r: other threads may be parsing too
        for (char* tok = strtok_r(buf, ",", &save); tok; tok = strtok_r(nullptr, ",", &save)) {
            char* eq = strchr(tok, '=');
            if (!eq) continue;
            *eq = '\0';
            const char* v = eq + 1;
            if (!strcmp(tok, "kernel")) t.kernel = !strcmp(v, "direct") ? 1 : !strcmp(v, "window") ? 2 : 0;
            else if (!strcmp(tok, "gb")) t.gb = atoi(v);
            else if (!strcmp(tok, "th")) t.th = atoi(v);
            else if (!strcmp(tok, "tw")) t.tw = atoi(v);
            else if (!strcmp(tok, "r")) t.r = atoi(v);
            else if (!strcmp(tok, "block")) t.block = atoi(v);
            else if (!strcmp(tok, "full")) t.full = atoi(v);
            else if (!strcmp(tok, "pitch_add")) t.pitch_add = atoi(v);
            else if (!strcmp(tok, "coal")) t.coal = atoi(v);
            else if (!strcmp(tok, "split")) t.split = atoi(v);
            else if (!strcmp(tok, "share")) t.share = atoi(v);
        }
    }
    return t;
}

int elem_bytes(int dtype) { return dtype == DCNV4_F32 ? 4 : 2; }

// Fewest output rows per band when bands are added to fill the GPU.
constexpr int kMinBandRows = 7;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Window extent (pixels, clamped to the zero-bordered image) for `tile`
// outputs along one axis with margin r.
int window_extent(int tile, int stride, int K, int dil, int r, int in)
{
    const int64_t e = (int64_t)(tile - 1) * stride + (int64_t)(K - 1) * dil + 2 + 2 * (int64_t)r;
    return (int)(e < in + 2 ? e : in + 2);
}

// LDS row pitch (16-byte entries): the window's ww pixels plus at least two
// zero columns, rounded up to 16 entries so that moving one row down keeps a
// lane on the same LDS banks.
int pitch_for(int ww) { return (ww + 2 + 15) / 16 * 16 + tune().pitch_add; }

// LDS bytes of a window of GB groups with `unit` bytes per group and pixel.
int lds_for(int wh, int ww, int slot)
{
    return wh * pitch_for(ww) * slot;
}

// Threads per workgroup for `units` lanes of work: the most the kernel allows
// (more waves per CU hide more latency; measured faster than the smallest
// block with the same number of passes), or the smallest multiple of 64 that
// covers the units in one pass.
int pick_block(int64_t units, int max_block)
{
    const int64_t b = ceil_div(units, 64) * 64;
    return (int)(b < max_block ? b : max_block);
}

bool plan_window(const Problem& p, Plan* pl)
{
    const Tune& t = tune();
    const int s = elem_bytes(p.dtype);
    if (p.K != 3 || (p.Cg * s) % 16) return false;
    const int nv = p.Cg * s / 16;
    if (nv < 1 || nv > 5) return false;
    if ((uintptr_t)p.x % 16 || (uintptr_t)p.out % 16) return false;
    const int ub = p.Cg * s;                   // bytes of one group of one pixel
    int R = t.r >= 0 ? t.r : 5;                // margin for the offsets, pixels
    // units of three or more vectors: one lane per vector (whole-unit lanes
    // need so many registers that a workgroup is capped at 512 threads)
    int lpu = (t.split == 1 && nv > 1) || (t.split < 0 && nv >= 3) ? nv : 1;
    const int cus = p.cus;

    // group blocks to try, smallest first (all divisors of G unless tuned)
    int order[64], no = 0;
    for (int gb = 1; gb <= p.G && no < 64; ++gb)
        if (p.G % gb == 0 && (!t.gb || gb == t.gb)) order[no++] = gb;
    if (!no) return false;

    int GB = 0, TH = 0, TW = 0, WH = 0, WW = 0, full = 0;
    // the whole zero-bordered image: no point can leave it
    if (t.full != 0) {
        for (int oi = 0; oi < no; ++oi) {
            const int gb = order[oi];
            if (lds_for(p.H + 2, p.W + 2, gb * ub) > kLdsPerCu) break;
            GB = gb;
            if ((int64_t)p.Ho * p.Wo * gb >= 128) break;
        }
        if (GB) { full = 1; TH = p.Ho; TW = p.Wo; WH = p.H + 2; WW = p.W + 2; }
    }
    // bands of full-width rows: the band height for margin r and groups gb
    // that minimises (rounds of workgroups) x (rows computed + half the rows
    // staged); false when no band fits or too many are needed
    auto band_plan = [&](int gb, int r, int* th_out, int64_t* rounds_out) {
        const int slot = gb * ub;
        const int ww = window_extent(t.tw ? t.tw : p.Wo, p.stride, p.K, p.dil, r, p.W);
        int max_th = 0;
        for (int th = 1; th <= p.Ho; ++th) {
            if (lds_for(window_extent(th, p.stride, p.K, p.dil, r, p.H), ww, slot) > kLdsPerCu) break;
            max_th = th;
        }
        if (t.th) max_th = t.th;
        if (max_th < 1) return false;
        const int nb0 = (int)ceil_div(p.Ho, max_th);
        if (nb0 > (lpu > 1 ? 8 : 4) && !t.th) return false;
        double best = 1e30;
        for (int nb = nb0; nb <= 2 * nb0; ++nb) {
            const int th = (int)ceil_div(p.Ho, nb);
            const int64_t wgs = (int64_t)p.N * ceil_div(p.Ho, th) * (p.G / gb);
            const int64_t rounds = ceil_div(wgs, cus);
            const double cost = (double)rounds * (th + 0.5 * window_extent(th, p.stride, p.K, p.dil, r, p.H));
            if (cost < best) { best = cost; *th_out = th; *rounds_out = rounds; }
        }
        return true;
    };
    for (int oi = 0; oi < no && !GB && t.full != 1; ++oi) {
        int th = 0;
        int64_t rounds = 0;
        if (!band_plan(order[oi], R, &th, &rounds)) continue;
        // one pixel less of margin when that saves a whole round of
        // workgroups (stage-1 fp32: two bands of 28 rows with margin 4,
        // 60.3 us, against three of 19 with margin 5, 62.6 us).  A smaller
        // margin sends more points to the global fallback, so it is not
        // taken otherwise (the latent shape with margin 4: 54.6 against
        // 52.5 us at the same band count)
        int th4 = 0;
        int64_t rounds4 = 0;
        if (t.r < 0 && R > 1 && band_plan(order[oi], R - 1, &th4, &rounds4) && rounds4 < rounds) {
            th = th4;
            R = R - 1;
        }
        GB = order[oi]; TH = th; TW = t.tw ? t.tw : p.Wo;
    }
    // tiles of 16 x 64 outputs with a 12-pixel margin, one lane per vector,
    // when rows are too wide for bands (the 256x256 shape: 126 against 179 us
    // for the direct kernel with its 8-pixel offsets, which send a third of
    // the units to the fallback; smaller offsets fall back less)
    if (!GB && t.full != 1 && nv >= 2) {
        const int R2 = t.r >= 0 ? t.r : 12;
        const int th = t.th ? t.th : 16, tw = t.tw ? t.tw : 64;
        for (int oi = 0; oi < no && !GB; ++oi) {
            const int gb = order[oi];
            if (lds_for(window_extent(th, p.stride, p.K, p.dil, R2, p.H),
                        window_extent(tw, p.stride, p.K, p.dil, R2, p.W), gb * ub) > kLdsPerCu)
                continue;
            GB = gb; TH = th; TW = tw; R = R2;
            if (t.split != 0) lpu = nv;
        }
    }
    if (!GB) return false;
    // fill the GPU: each workgroup holds one CU for the whole of its tile, so
    // a plan with fewer workgroups than CUs leaves CUs idle.  Full-width plans
    // take more bands; bands under kMinBandRows rows cost more in margins than
    // they save, and there the direct kernel is faster (measured at batch 1 to
    // 32 of the stage-1 shape and 1 to 4 of the latent shape)
    if (t.kernel == 0 && t.full < 0 && !t.th && !t.tw && !t.gb) {
        const int64_t per_band = (int64_t)p.N * ceil_div(p.Wo, TW) * (p.G / GB);
        if (per_band * ceil_div(p.Ho, TH) < cus) {
            if (TW < p.Wo) return false;
            const int th = (int)ceil_div(p.Ho, ceil_div(cus, per_band));
            if (th < kMinBandRows) return false;
            if (full) {
                full = 0;
                R = t.r >= 0 ? t.r : 5;
            }
            TH = th;
        }
    }
    if (!full) {
        if (TH > p.Ho) TH = p.Ho;
        if (TW > p.Wo) TW = p.Wo;
        WH = window_extent(TH, p.stride, p.K, p.dil, R, p.H);
        WW = window_extent(TW, p.stride, p.K, p.dil, R, p.W);
    }
    const int slot = GB * ub;
    const int lds = lds_for(WH, WW, slot);
    if (lds > kLdsPerCu) return false;
    const int64_t units = (int64_t)TH * TW * GB;
    const int64_t items = units * lpu;
    const int max_block = lpu > 1 ? 1024 : window_max_block(nv);
    int block = t.block ? t.block : pick_block(items, max_block);
    if (block < 64 || block % 64 || block > max_block) block = max_block;
    if (ceil_div(items, block) > 64) return false;   // the kernel tracks at most 64 passes

    // offset rows through LDS: needs evenly spaced rows of one group (GB = 1,
    // full-width tiles, rows a whole number of dwords apart) and room for the
    // per-wave buffers
    const int s_el = elem_bytes(p.dtype);
    const bool coal_ok = lpu == 1 && GB == 1 && TW == p.Wo && (p.off_row * s_el) % 4 == 0 &&
                         p.off_row * s_el < (1 << 24) &&
                         lds + window_coal_lds_bytes(block, p.dtype, p.P) <= kLdsPerCu;
    pl->coal = t.coal == 0 ? 0 : coal_ok ? 1 : 0;
    pl->lds_total = lds + (pl->coal ? window_coal_lds_bytes(block, p.dtype, p.P) : 0);

    pl->kernel = kKernelWindow;
    pl->vec = 16;
    pl->lanes = lpu;
    pl->lpu = lpu;
    // point coefficients shared over a unit's lanes: four lanes (stage-1 fp32:
    // 67.1 us against 74.0 without); two lanes measured slower (the 256x256
    // bf16 shape: 126.2 against 122.2 us), so only on request; one group per
    // workgroup (the kernel's corner reads step over a pixel's vectors with a
    // constant offset)
    pl->share = GB == 1 && ((lpu == 4 && t.share != 0) || (lpu == 2 && t.share == 1)) ? 1 : 0;
    pl->block = block;
    pl->nv = nv;
    pl->GB = GB; pl->TH = TH; pl->TW = TW; pl->RY = full ? 0 : R; pl->RX = full ? 0 : R;
    pl->WH = WH; pl->WW = WW; pl->full = full;
    pl->lds_bytes = lds;
    pl->grid = (int64_t)p.N * ceil_div(p.Ho, TH) * ceil_div(p.Wo, TW) * (p.G / GB);
    return true;
}

void plan_direct(const Problem& p, Plan* pl)
{
    const int s = elem_bytes(p.dtype);
    // widest read (<= 16 bytes) that divides the group's channel bytes and
    // keeps x and out reads/writes aligned
    int vb = 16;
    while (vb > s) {
        if ((p.Cg * s) % vb == 0 && (uintptr_t)p.x % vb == 0 && (uintptr_t)p.out % vb == 0) break;
        vb >>= 1;
    }
    pl->kernel = kKernelDirect;
    pl->vec = vb;
    pl->lanes = p.Cg * s / vb;
    pl->block = 256;
    pl->nv = 0;
    pl->GB = pl->TH = pl->TW = pl->RY = pl->RX = pl->WH = pl->WW = pl->full = 0;
    pl->coal = 0;
    pl->lds_total = 0;
    pl->lds_bytes = 0;
    pl->lpu = 1;
    pl->share = 0;
    const int64_t lanes_img = (int64_t)p.Ho * p.Wo * p.G * pl->lanes;
    pl->grid = (int64_t)p.N * ceil_div(lanes_img, 256);
}

}  // namespace

void make_plan(const Problem& p, Plan* plan)
{
    const Tune& t = tune();
    if (t.kernel != 1 && plan_window(p, plan)) return;
    plan_direct(p, plan);
}

hipError_t launch_forward(const Problem& p, const Plan& plan, hipStream_t stream)
{
    const int s = elem_bytes(p.dtype);
    KArgs a;
    memset(&a, 0, sizeof a);
    a.x = p.x; a.off = p.off; a.msk = p.msk; a.out = p.out;
    a.H = p.H; a.W = p.W; a.G = p.G; a.Cg = p.Cg; a.C = p.G * p.Cg;
    a.K = p.K; a.P = p.P; a.stride = p.stride; a.pad = p.pad; a.dil = p.dil;
    a.Ho = p.Ho; a.Wo = p.Wo; a.remove_center = p.remove_center; a.softmax = p.softmax;
    a.off_row = p.off_row; a.mask_row = p.mask_row;
    a.offset_scale = p.offset_scale;
    a.img_x_elems = (int64_t)p.H * p.W * a.C;
    a.img_out_elems = (int64_t)p.Ho * p.Wo * a.C;
    a.img_off_elems = (int64_t)p.Ho * p.Wo * p.off_row;
    a.img_mask_elems = (int64_t)p.Ho * p.Wo * p.mask_row;
    a.img_x_bytes = (uint32_t)(a.img_x_elems * s);
    // an image's offset/weight rows end with its last pixel's used elements;
    // rounded up to whole dwords (a dword holding a used byte is never past
    // the allocation's last page)
    a.img_off_bytes = (uint32_t)(((((int64_t)p.Ho * p.Wo - 1) * p.off_row + (int64_t)p.G * 2 * p.P) * s + 3) & ~3ll);
    a.img_mask_bytes = (uint32_t)(((((int64_t)p.Ho * p.Wo - 1) * p.mask_row + (int64_t)p.G * p.P) * s + 3) & ~3ll);

    if (plan.kernel == kKernelDirect) {
        a.lanes = plan.lanes;
        a.vec_bytes = plan.vec;
        a.units_img = (uint32_t)((int64_t)p.Ho * p.Wo * p.G);
        a.blocks_per_image = (uint32_t)ceil_div((int64_t)a.units_img * plan.lanes, 256);
        a.div_lanes = make_fastdiv((uint32_t)plan.lanes);
        a.div_G = make_fastdiv((uint32_t)p.G);
        a.div_Wo = make_fastdiv((uint32_t)p.Wo);
        return launch_direct(a, p.dtype, plan.block, (int64_t)a.blocks_per_image * p.N, stream);
    }
    a.GB = plan.GB; a.TH = plan.TH; a.TW = plan.TW; a.RY = plan.RY; a.RX = plan.RX;
    if (plan.full) a.RY = a.RX = p.H + p.W + 2;   // window origin clamps to (-1, -1)
    a.WH = plan.WH; a.WW = plan.WW; a.full = plan.full; a.coal = plan.coal;
    a.pitch = pitch_for(plan.WW);
    a.slot_bytes = plan.GB * p.Cg * s;
    a.tiles_y = (uint32_t)ceil_div(p.Ho, plan.TH);
    a.tiles_x = (uint32_t)ceil_div(p.Wo, plan.TW);
    a.gtiles = (uint32_t)(p.G / plan.GB);
    a.div_GB = make_fastdiv((uint32_t)plan.GB);
    a.div_TW = make_fastdiv((uint32_t)plan.TW);
    a.div_tiles_x = make_fastdiv(a.tiles_x);
    a.div_tiles_y = make_fastdiv(a.tiles_y);
    a.div_gtiles = make_fastdiv(a.gtiles);
    a.div_CPS = make_fastdiv((uint32_t)(plan.GB * plan.nv));
    a.div_pitch = make_fastdiv((uint32_t)a.pitch);
    a.win_bytes = (uint32_t)plan.lds_bytes;
    a.lds_bytes = (uint32_t)plan.lds_total;
    a.lpu = plan.lpu;
    a.share = plan.share;
    a.nvt = plan.nv;
    a.div_lpu = make_fastdiv((uint32_t)plan.lpu);
    return p.softmax ? launch_window_softmax(a, p.dtype, plan.nv, plan.block, plan.grid, stream)
                     : launch_window(a, p.dtype, plan.nv, plan.block, plan.grid, stream);
}

}  // namespace dcnv4

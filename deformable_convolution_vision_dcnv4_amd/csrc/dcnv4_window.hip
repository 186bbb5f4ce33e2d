// DCNv4 forward, window kernel family (kernel template: dcnv4_window_impl.h):
// the DCNv4 aggregation with raw, signed dynamic weights (jsqmd.com/news/933833
// section 1, first optimisation; bqwf.cn/news/1148139 section 2.1), and the
// planner's window constants.

#include "dcnv4_window_impl.h"

namespace dcnv4 {

int window_max_block(int nv) { return nv <= 2 ? 1024 : 512; }

int window_coal_lds_bytes(int block, int dtype, int P)
{
    const int s = dtype == DCNV4_F32 ? 4 : 2;
    return block * (2 * P * s / 4) * 4;
}

hipError_t launch_window(const KArgs& a, int dtype, int nv, int block, int64_t grid, hipStream_t stream)
{
    return launch_window_form<0>(a, dtype, nv, block, grid, stream);
}

}  // namespace dcnv4

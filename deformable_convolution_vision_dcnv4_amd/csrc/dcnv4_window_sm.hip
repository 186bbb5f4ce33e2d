// DCNv3-style aggregation on the window kernel family (kernel template:
// dcnv4_window_impl.h): each (pixel, group)'s P weights pass through a
// softmax before the sampling, the normalisation DCNv4 removes
// (jsqmd.com/news/933833 section 1, first optimisation; bqwf.cn/news/1148139
// section 2.1), kept for comparing the two on the same kernel.

#include "dcnv4_window_impl.h"

namespace dcnv4 {

hipError_t launch_window_softmax(const KArgs& a, int dtype, int nv, int block, int64_t grid, hipStream_t stream)
{
    return launch_window_form<1>(a, dtype, nv, block, grid, stream);
}

}  // namespace dcnv4

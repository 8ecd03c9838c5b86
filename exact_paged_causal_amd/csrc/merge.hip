// merge.hip -- the log-sum-exp merge pass: one wave per output row
// (merge_row.h), after the split-KV folds and after the tiled prefills' key
// splits.  A merge inside the folds (the last work item of each row chunk,
// found through a counter) was built and measured slower: every work item
// then needs a device-scope release fence before it counts, which on this
// multi-XCD part writes back its L2.
#include "merge_row.h"

namespace atlas {
namespace {

template <int D, int NF>
__global__ __launch_bounds__(64) void merge_kernel(SplitArgs a)
{
    // 32-bit index arithmetic: the grid has fewer than 2^31 rows.
    const uint32_t row = blockIdx.x;
    const uint32_t bi = row / (uint32_t)a.hq;
    const int h = (int)(row - bi * (uint32_t)a.hq);
    const uint32_t b32 = bi / (uint32_t)a.q_len;
    const int i = (int)(bi - b32 * (uint32_t)a.q_len);
    const int b = (int)b32;
    const int64_t row_id = row;
    merge_row<D, NF>(a, row_id, [&] { return merge_split_count(a, b, i, h); }, threadIdx.x);
}

}  // namespace

hipError_t launch_merge(const SplitArgs &a, hipStream_t stream)
{
    const int64_t rows = (int64_t)a.batch * a.q_len * a.hq;
    if (rows <= 0 || rows > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    // The first batch of accumulator rows covers max_splits (up to 64).
    const int nf = a.max_splits <= 8 ? 0 : a.max_splits <= 16 ? 1 : a.max_splits <= 32 ? 2 : 3;
    void (*kernel)(SplitArgs);
    if (a.head_dim == 64) {
        void (*const k64[4])(SplitArgs) = {merge_kernel<64, 8>, merge_kernel<64, 16>, merge_kernel<64, 32>,
                                           merge_kernel<64, 64>};
        kernel = k64[nf];
    } else {
        void (*const k128[4])(SplitArgs) = {merge_kernel<128, 8>, merge_kernel<128, 16>, merge_kernel<128, 32>,
                                            merge_kernel<128, 64>};
        kernel = k128[nf];
    }
    hipLaunchKernelGGL(kernel, dim3((unsigned)rows), dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace atlas

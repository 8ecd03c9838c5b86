// merge.hip -- the log-sum-exp merge pass: one wave per output row
// (merge_row.h), after the split-KV folds and after the tiled prefills' key
// splits.  A merge inside the folds (the last work item of each row chunk,
// found through a counter) was built and measured slower: every work item
// then needs a device-scope release fence before it counts, which on this
// multi-XCD part writes back its L2.
#include "merge_row.h"

namespace atlas {
namespace {

template <int D>
__global__ __launch_bounds__(64) void merge_kernel(SplitArgs a)
{
    const int64_t row_id = blockIdx.x;
    const int h = (int)(row_id % a.hq);
    const int64_t bi = row_id / a.hq;
    const int i = (int)(bi % a.q_len);
    const int b = (int)(bi / a.q_len);
    merge_row<D>(a, row_id, merge_split_count(a, b, i, h), threadIdx.x);
}

}  // namespace

hipError_t launch_merge(const SplitArgs &a, hipStream_t stream)
{
    const int64_t rows = (int64_t)a.batch * a.q_len * a.hq;
    if (a.head_dim == 64)
        hipLaunchKernelGGL(merge_kernel<64>, dim3((unsigned)rows), dim3(64), 0, stream, a);
    else
        hipLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)rows), dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace atlas

// merge.hip -- the log-sum-exp merge pass after the split-KV folds and after
// the tiled prefills' key splits: one wave per output row (merge_row.h) for
// up to 64 splits, eight waves per row past that.  A merge inside the folds (the last work item of each row chunk,
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

// Rows with more than 64 splits (a few rows over long contexts, which the
// plan spreads over many splits to fill the chip): one wave walking the
// splits would make a chain of n / 32 memory round trips, so eight waves
// share each row.  All threads take the maximum and the denominator over
// strided splits; wave w sums the weighted accumulator rows of the w-th
// contiguous eighth of the splits in order, and the eight partial rows are
// added in wave order.  Every step has a fixed order, so the result does
// not depend on scheduling.
template <int D>
__global__ __launch_bounds__(512) void merge_wide_kernel(SplitArgs a)
{
    constexpr int NW = 8;          // waves per row
    constexpr int DPT = D / 64;    // dims per lane
    constexpr int kBatch = 16;     // accumulator rows loaded together per wave
    __shared__ float red[NW];
    __shared__ float part[NW][D];
    const uint32_t row = blockIdx.x;
    const uint32_t bi = row / (uint32_t)a.hq;
    const int h = (int)(row - bi * (uint32_t)a.hq);
    const uint32_t b32 = bi / (uint32_t)a.q_len;
    const int i = (int)(bi - b32 * (uint32_t)a.q_len);
    const int b = (int)b32;
    const int64_t row_id = row;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int ms = a.max_splits;
    const float *ml = a.ws_ml + row_id * ms * 2;
    const float *acc = a.ws_acc + row_id * ms * D;
    int n = merge_split_count(a, b, i, h);
    n = n < ms ? n : ms;  // the workspace holds max_splits states per row

    float mm = -INFINITY;
    for (int s = tid; s < n; s += NW * 64)
        mm = fmaxf(mm, ml[2 * s]);
    for (int off = 32; off > 0; off >>= 1)
        mm = fmaxf(mm, __shfl_xor(mm, off));
    if (lane == 0)
        red[wv] = mm;
    __syncthreads();
    mm = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w)
        mm = fmaxf(mm, red[w]);
    const float msafe = mm == -INFINITY ? 0.0f : mm;
    __syncthreads();  // red is written again below

    float L = 0.0f;
    for (int s = tid; s < n; s += NW * 64)
        L = fmaf(ml[2 * s + 1], fast_exp2(ml[2 * s] - msafe), L);
    for (int off = 32; off > 0; off >>= 1)
        L += __shfl_xor(L, off);
    if (lane == 0)
        red[wv] = L;

    const int per = (n + NW - 1) / NW;
    const int s_lo = wv * per;
    const int s_hi = s_lo + per < n ? s_lo + per : n;
    float o[DPT];
#pragma unroll
    for (int e = 0; e < DPT; ++e)
        o[e] = 0.0f;
    for (int s0 = s_lo; s0 < s_hi; s0 += 64) {
        const int cnt = s_hi - s0 < 64 ? s_hi - s0 : 64;
        const float fl = lane < cnt ? fast_exp2(ml[2 * (s0 + lane)] - msafe) : 0.0f;
        for (int b0 = 0; b0 < cnt; b0 += kBatch) {
            float v[kBatch][DPT];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                // Past this wave's last split the load repeats it (in bounds, unused).
                const int s = s0 + (b0 + j < cnt ? b0 + j : cnt - 1);
#pragma unroll
                for (int e = 0; e < DPT; ++e)
                    v[j][e] = acc[(int64_t)s * D + e * 64 + lane];
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                if (b0 + j < cnt) {
                    const float f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fl), b0 + j));
#pragma unroll
                    for (int e = 0; e < DPT; ++e)
                        o[e] = fmaf(v[j][e], f, o[e]);
                }
            }
        }
    }
#pragma unroll
    for (int e = 0; e < DPT; ++e)
        part[wv][e * 64 + lane] = o[e];
    __syncthreads();
    L = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w)
        L += red[w];
    if (tid < D) {
        float sum = part[0][tid];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            sum += part[w][tid];
        float *orow = a.out + row_id * D;
        if (L > 0.0f) {
            orow[tid] = sum * (1.0f / L);
            if (a.lse && tid == 0)
                a.lse[row_id] = (mm + log2f(L)) * kLn2;
        } else {
            orow[tid] = __builtin_nanf("");
            if (a.lse && tid == 0)
                a.lse[row_id] = -INFINITY;
        }
    }
}

}  // namespace

hipError_t launch_merge(const SplitArgs &a, hipStream_t stream)
{
    const int64_t rows = (int64_t)a.batch * a.q_len * a.hq;
    if (rows <= 0 || rows > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    if (a.max_splits > 64) {
        if (a.head_dim == 64)
            hipLaunchKernelGGL(merge_wide_kernel<64>, dim3((unsigned)rows), dim3(512), 0, stream, a);
        else
            hipLaunchKernelGGL(merge_wide_kernel<128>, dim3((unsigned)rows), dim3(512), 0, stream, a);
        return hipGetLastError();
    }
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

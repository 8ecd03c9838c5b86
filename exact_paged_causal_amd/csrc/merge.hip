// merge.hip -- exact log-sum-exp merge of the split-KV partial states.
//
// For one output row (sequence b, query i, q-head h) the splits s = 0..n-1
// left (m_s, l_s, acc_s) with m_s in log2 units.  With M = max m_s:
//     L   = sum_s l_s 2^(m_s - M)
//     out = sum_s acc_s 2^(m_s - M) / L
//     lse = (M + log2 L) ln 2
// A split whose keys are all masked for this row has l_s = 0, m_s = -inf and
// drops out.  The splits are visited in a fixed order, so the result does
// not depend on scheduling (CPUAttn README "Operator model": split-K only
// with a structured merge; CFR-Atlas "Core contract": folded == full K/V).
// The number of splits is recomputed from the same plan the split kernels
// used (plan.h), so no count has to travel through memory.
#include "device.h"
#include "kernels.h"

namespace atlas {
namespace {

template <int D>
__global__ __launch_bounds__(64) void merge_kernel(SplitArgs a)
{
    constexpr int DPT = D / 64;  // dims per lane
    extern __shared__ float s_f[];  // [max_splits] weights of the splits
    const int lane = threadIdx.x;
    const int64_t row_id = blockIdx.x;
    const int h = (int)(row_id % a.hq);
    const int64_t bi = row_id / a.hq;
    const int i = (int)(bi % a.q_len);
    const int b = (int)(bi / a.q_len);
    const int g = a.groups.group_of[h];
    const int gsize = a.groups.start[g + 1] - a.groups.start[g];
    const int rr = i * gsize + a.groups.slot_of[h];

    int ctx = a.context_lens[b];
    ctx = ctx < 0 ? 0 : (ctx > a.max_context ? a.max_context : ctx);
    const ChunkRows cr = chunk_rows(rr / a.rows_per_item, a.rows_per_item, gsize, a.q_len, ctx);
    const int W = a.window ? a.window[b] : 0;
    const int S = a.sinks ? a.sinks[b] : 0;
    int n;
    if (a.tiled_blocks > 0) {
        // Key splits of the tiled prefill: this query's block of positions.
        const int i0 = (i / a.tiled_npos) * a.tiled_npos;
        const int i1 = i0 + a.tiled_npos < a.q_len ? i0 + a.tiled_npos : a.q_len;
        const int pos_lo = ctx - a.q_len + i0;
        const int pos_hi = ctx - a.q_len + i1 - 1;
        const int key_hi = (a.mods.any && !a.mods.causal) ? (pos_hi >= 0 ? ctx - 1 : -1) : pos_hi;
        const TiledBlocks tb = tiled_blocks(pos_lo, key_hi, W, W > 0 ? S : 0, 64);
        n = (tb.n + a.tiled_blocks - 1) / a.tiled_blocks;
    } else {
        // Non-causal rows (atlas_attend_mods) were planned over [0, ctx).
        const SplitPlan plan = (a.mods.any && !a.mods.causal) ? plan_splits(ctx - 1, ctx - 1, 0, 0, a.split_tokens)
                                                              : plan_splits(cr.pos_min, cr.pos_max, W, S,
                                                                            a.split_tokens);
        n = plan.n_splits;
    }

    const float *ml = a.ws_ml + row_id * a.max_splits * 2;
    const float *acc = a.ws_acc + row_id * a.max_splits * D;

    // Pass 1 (lanes over splits): the maximum, then each split's weight.
    float mm = -INFINITY;
    for (int s = lane; s < n; s += 64)
        mm = fmaxf(mm, ml[2 * s]);
    for (int off = 32; off > 0; off >>= 1)
        mm = fmaxf(mm, __shfl_xor(mm, off));
    const float msafe = mm == -INFINITY ? 0.0f : mm;
    float L = 0.0f;
    for (int s = lane; s < n; s += 64) {
        const float f = fast_exp2(ml[2 * s] - msafe);
        s_f[s] = f;
        L = fmaf(ml[2 * s + 1], f, L);
    }
    for (int off = 32; off > 0; off >>= 1)
        L += __shfl_xor(L, off);
    __syncthreads();

    // Pass 2 (lanes over dims): weighted sum of the accumulators, in split order.
    float o[DPT];
#pragma unroll
    for (int e = 0; e < DPT; ++e)
        o[e] = 0.0f;
#pragma unroll 8
    for (int s = 0; s < n; ++s) {
        const float f = s_f[s];
#pragma unroll
        for (int e = 0; e < DPT; ++e)
            o[e] = fmaf(acc[(int64_t)s * D + e * 64 + lane], f, o[e]);
    }
    float *orow = a.out + row_id * D;
    if (L > 0.0f) {
        const float inv = 1.0f / L;
#pragma unroll
        for (int e = 0; e < DPT; ++e)
            orow[e * 64 + lane] = o[e] * inv;
        if (a.lse && lane == 0)
            a.lse[row_id] = (mm + log2f(L)) * kLn2;
    } else {
#pragma unroll
        for (int e = 0; e < DPT; ++e)
            orow[e * 64 + lane] = __builtin_nanf("");
        if (a.lse && lane == 0)
            a.lse[row_id] = -INFINITY;
    }
}

}  // namespace

hipError_t launch_merge(const SplitArgs &a, hipStream_t stream)
{
    const int64_t rows = (int64_t)a.batch * a.q_len * a.hq;
    const size_t lds = sizeof(float) * (size_t)a.max_splits;
    if (a.head_dim == 64)
        hipLaunchKernelGGL(merge_kernel<64>, dim3((unsigned)rows), dim3(64), lds, stream, a);
    else
        hipLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)rows), dim3(64), lds, stream, a);
    return hipGetLastError();
}

}  // namespace atlas

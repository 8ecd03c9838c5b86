// merge_row.h -- exact log-sum-exp merge of one output row's split states
// (one wave per row), used by the merge kernel (merge.hip).
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
#pragma once

#include "device.h"
#include "kernels.h"

namespace atlas {

// Splits of output row (b, i, h) (a wave-uniform value).
__device__ __forceinline__ int merge_split_count(const SplitArgs &a, int b, int i, int h)
{
    const int g = a.groups.group_of[h];
    const int gsize = a.groups.start[g + 1] - a.groups.start[g];
    const int rr = i * gsize + a.groups.slot_of[h];
    int ctx = a.context_lens[b];
    ctx = ctx < 0 ? 0 : (ctx > a.max_context ? a.max_context : ctx);
    const int W = a.window ? a.window[b] : 0;
    const int S = a.sinks ? a.sinks[b] : 0;
    if (a.tiled_blocks > 0) {
        // Key splits of the tiled prefill: this query's block of positions.
        const int i0 = (i / a.tiled_npos) * a.tiled_npos;
        const int i1 = i0 + a.tiled_npos < a.q_len ? i0 + a.tiled_npos : a.q_len;
        const int pos_lo = ctx - a.q_len + i0;
        const int pos_hi = ctx - a.q_len + i1 - 1;
        const int key_hi = (a.mods.any && !a.mods.causal) ? (pos_hi >= 0 ? ctx - 1 : -1) : pos_hi;
        const TiledBlocks tb = tiled_blocks(pos_lo, key_hi, W, W > 0 ? S : 0, 64);
        return (tb.n + a.tiled_blocks - 1) / a.tiled_blocks;
    }
    // Non-causal rows (atlas_attend_mods) were planned over [0, ctx).
    const ChunkRows cr = chunk_rows(rr / a.rows_per_item, a.rows_per_item, gsize, a.q_len, ctx);
    const SplitPlan plan = (a.mods.any && !a.mods.causal) ? plan_splits(ctx - 1, ctx - 1, 0, 0, a.split_tokens)
                                                          : plan_splits(cr.pos_min, cr.pos_max, W, S, a.split_tokens);
    return plan.n_splits;
}

// One wave merges output row row_id = (b * q_len + i) * hq + h over its n
// splits: lanes over splits for the maximum and the denominator, then lanes
// over dims for the weighted sum in split order (each split's weight is the
// same hardware exponential both times).
template <int D>
__device__ __forceinline__ void merge_row(const SplitArgs &a, int64_t row_id, int n, int lane)
{
    constexpr int DPT = D / 64;  // dims per lane
    const float *ml = a.ws_ml + row_id * a.max_splits * 2;
    const float *acc = a.ws_acc + row_id * a.max_splits * D;

    float mm = -INFINITY;
    for (int s = lane; s < n; s += 64)
        mm = fmaxf(mm, ml[2 * s]);
    for (int off = 32; off > 0; off >>= 1)
        mm = fmaxf(mm, __shfl_xor(mm, off));
    const float msafe = mm == -INFINITY ? 0.0f : mm;
    float L = 0.0f;
    for (int s = lane; s < n; s += 64)
        L = fmaf(ml[2 * s + 1], fast_exp2(ml[2 * s] - msafe), L);
    for (int off = 32; off > 0; off >>= 1)
        L += __shfl_xor(L, off);

    float o[DPT];
#pragma unroll
    for (int e = 0; e < DPT; ++e)
        o[e] = 0.0f;
#pragma unroll 8
    for (int s = 0; s < n; ++s) {
        const float f = fast_exp2(ml[2 * s] - msafe);
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

}  // namespace atlas

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

// A call whose plan gives every row one split (max_splits == 1) needs no
// merge: the fold writes each row's final output and lse itself, with the
// merge's own arithmetic for a single split (its weight 2^0 = 1, its sum L =
// l), so the bits are those the merge would write.  l = 0 (nothing visible)
// gives NaN and lse = -inf.
__device__ __forceinline__ void write_single_split(const SplitArgs &a, int64_t row_id, int d, float m, float l,
                                                   float acc)
{
    const bool any = l > 0.0f;
    a.out[row_id * a.head_dim + d] = any ? acc * (1.0f / l) : __builtin_nanf("");
    if (d == 0 && a.lse)
        a.lse[row_id] = any ? (m + log2f(l)) * kLn2 : -INFINITY;
}

// One wave merges output row row_id = (b * q_len + i) * hq + h over its n
// splits: lanes over splits for the maximum and the denominator, then lanes
// over dims for the weighted sum in split order (each split's weight is the
// same hardware exponential both times).  The chain of memory round trips is
// kept short: the (m, l) pairs of the first 64 splits (one per lane) and
// the accumulator rows of the first NF are loaded before the split count is
// known (their addresses depend only on the row; entries past the count are
// never used), the weights are broadcast from the lanes that computed them,
// and any further splits are loaded 32 at a time.  count() gives the split
// count; NF (8 to 64) is chosen on the host to cover max_splits.
template <int D, int NF, class Count>
__device__ __forceinline__ void merge_row(const SplitArgs &a, int64_t row_id, Count count, int lane)
{
    static_assert(NF >= 1 && NF <= 64, "the first batch is at most one split per lane");
    constexpr int DPT = D / 64;    // dims per lane
    constexpr int kBatch = 32;     // further accumulator rows loaded together
    const int ms = a.max_splits;
    const float *ml = a.ws_ml + row_id * ms * 2;
    const float *acc = a.ws_acc + row_id * ms * D;

    // Loads independent of the split count: (m, l) of splits 0..63 and the
    // accumulator rows of splits 0..NF-1 (clamped to the row's max_splits
    // slots).
    const int first = ms < 64 ? (ms > 0 ? ms : 0) : 64;
    float2 mlv = make_float2(-INFINITY, 0.0f);
    if (lane < first)
        mlv = *reinterpret_cast<const float2 *>(ml + 2 * lane);
    float v0[NF][DPT];
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
        for (int e = 0; e < DPT; ++e)
            v0[j][e] = 0.0f;
    if (first > 0) {
#pragma unroll
        for (int j = 0; j < NF; ++j) {
            const int sj = j < first ? j : first - 1;
#pragma unroll
            for (int e = 0; e < DPT; ++e)
                v0[j][e] = acc[(int64_t)sj * D + e * 64 + lane];
        }
    }
    int n = count();
    n = n < ms ? n : ms;  // the workspace holds max_splits states per row

    const float m0 = lane < n ? mlv.x : -INFINITY;
    const float l0 = lane < n ? mlv.y : 0.0f;
    float mm = m0;
    for (int s = lane + 64; s < n; s += 64)
        mm = fmaxf(mm, ml[2 * s]);
    for (int off = 32; off > 0; off >>= 1)
        mm = fmaxf(mm, __shfl_xor(mm, off));
    const float msafe = mm == -INFINITY ? 0.0f : mm;
    const float f0 = fast_exp2(m0 - msafe);
    float L = lane < n ? fmaf(l0, f0, 0.0f) : 0.0f;
    for (int s = lane + 64; s < n; s += 64)
        L = fmaf(ml[2 * s + 1], fast_exp2(ml[2 * s] - msafe), L);
    for (int off = 32; off > 0; off >>= 1)
        L += __shfl_xor(L, off);

    float o[DPT];
#pragma unroll
    for (int e = 0; e < DPT; ++e)
        o[e] = 0.0f;
    // Splits 0..NF-1 from the registers loaded above.
#pragma unroll
    for (int j = 0; j < NF; ++j) {
        if (j < n) {
            const float f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f0), j));
#pragma unroll
            for (int e = 0; e < DPT; ++e)
                o[e] = fmaf(v0[j][e], f, o[e]);
        }
    }
    // Further splits, 64 weights and kBatch rows at a time (the weights of
    // splits below 64 are the f0 computed above).
    for (int s0 = 0; s0 < n; s0 += 64) {
        const float fl = s0 == 0 ? f0 : (s0 + lane < n ? fast_exp2(ml[2 * (s0 + lane)] - msafe) : 0.0f);
        const int nb = n - s0 < 64 ? n - s0 : 64;
        for (int b0 = s0 == 0 ? NF : 0; b0 < nb; b0 += kBatch) {
            float v[kBatch][DPT];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                // Past the last split the load repeats it (in bounds, unused).
                const int s = s0 + (b0 + j < nb ? b0 + j : nb - 1);
#pragma unroll
                for (int e = 0; e < DPT; ++e)
                    v[j][e] = acc[(int64_t)s * D + e * 64 + lane];
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                if (b0 + j < nb) {
                    const float f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fl), b0 + j));
#pragma unroll
                    for (int e = 0; e < DPT; ++e)
                        o[e] = fmaf(v[j][e], f, o[e]);
                }
            }
        }
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

// split_valu.hip -- split-KV fold on the vector ALUs (fp32 K/V; bf16 runs on
// the matrix cores, split_mfma.hip).
//
// One workgroup (4 waves) = one work item (sequence b, K/V head g, chunk of
// rows, split s).  Its keys are the span plan.h assigns to split s; every
// visible key is folded, for every row of the chunk, into an online-softmax
// state (running max m, sum l, accumulator acc) -- CFR-Atlas README: each
// page is folded into online softmax; CPUAttn README "Operator model": a
// split is allowed because a structured merge (merge.hip) recombines it.
// When the plan gives every row one split (short contexts), the work item's
// state is the row's final state and the fold writes the output and lse
// itself, with the merge's own arithmetic (merge_row.h): no merge runs.
//
// Lane layout.  A K or V row of D elements is read by a group of R lanes
// (R = 16 for 256-byte rows, 8 for 128-byte rows), each lane loading NL
// 16-byte pieces; one load instruction of a wave therefore covers 64/R whole
// rows (1 KiB contiguous when they sit in one page).  Each lane keeps its
// slice of q and acc for every row of the chunk in registers.  Dot products
// are reduced across the R lanes with DPP row operations; exp2 runs on the
// hardware v_exp_f32 with the scale folded by log2(e).  Page ids of the
// split are staged once in LDS, so the per-key address math is scalar-free
// shifts and masks (page sizes are powers of two).  K/V loads are
// non-temporal (NT instances) when one row chunk covers every row of a K/V
// head, so each row is read once per pass; with several chunks the chunks
// re-read the same rows and ordinary loads keep them in cache, as do the
// REGEN and MODS instances (REGEN's cold keys re-read page 0).  Iterations
// whose keys
// every row of the item sees (no window, all at or before the rows'
// positions) skip the per-key visibility test.
//
// In-kernel regeneration (REGEN instances): page-table entries of -1 mark
// pages that are not stored; their keys' K and V values are produced at fold
// time by the page regenerator's generator (philox.h) for exactly this
// lane's dims -- a lane's 16-byte piece is one generator call of 4 dims --
// so the fold sees the same bits a regenerated scratch page would hold.
// Their loads still go out so that the prefetch stays unconditional, but all
// to one row (row 0 of page 0 for the item's K/V head), which stays in cache
// however many resident rows stream past it.
//
// Modifications (MODS instances, atlas_attend_mods): non-causal rows see
// every key of the context (the split plan then spans [0, L)); an ALiBi slope
// per q-head adds -slope |pos - j| to the logit after the softcap; mask bits
// hide keys per (row, key).
#include <type_traits>

#include "device.h"
#include "kernels.h"
#include "merge_row.h"
#include "philox.h"

namespace atlas {
namespace {

template <typename E>
struct Elem;

template <>
struct Elem<float> {
    static constexpr int kPer16 = 4;
    __device__ static void unpack(const uint4 &c, float *out)
    {
        out[0] = __uint_as_float(c.x);
        out[1] = __uint_as_float(c.y);
        out[2] = __uint_as_float(c.z);
        out[3] = __uint_as_float(c.w);
    }
};

template <typename E, int D, int MC, int KU, bool REGEN, bool MODS, bool NT>
__global__ __launch_bounds__(256) void split_valu_kernel(SplitArgs a)
{
    constexpr int EPC = Elem<E>::kPer16;                 // elements per 16-byte piece
    constexpr int ROWB = D * (int)sizeof(E);             // bytes per K/V row
    constexpr int R = ROWB / 16 >= 16 ? 16 : ROWB / 16;  // lanes per row
    constexpr int NL = ROWB / (R * 16);                  // pieces per lane per row
    constexpr int DPL = NL * EPC;                        // dims per lane
    constexpr int GPW = 64 / R;                          // row groups per wave
    constexpr int KPI = 4 * GPW * KU;                    // keys per iteration per workgroup
    static_assert(R == 8 || R == 16, "row group");

    __shared__ int32_t s_pid[kMaxSplitPages];
    __shared__ float s_m[4][MC];
    __shared__ float s_l[4][MC];
    __shared__ float s_acc[4][MC][D];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int grp = lane / R;
    const int li = lane % R;

    const int split = blockIdx.x;
    const int g = blockIdx.y / a.n_chunks;
    const int chunk = blockIdx.y - g * a.n_chunks;
    const int b = blockIdx.z;
    const int gstart = a.groups.start[g];
    const int gsize = a.groups.start[g + 1] - gstart;

    int ctx = a.context_lens[b];
    ctx = ctx < 0 ? 0 : (ctx > a.max_context ? a.max_context : ctx);
    const ChunkRows cr = chunk_rows(chunk, MC, gsize, a.q_len, ctx);
    if (cr.r0 >= cr.r1)
        return;
    const int W = a.window ? a.window[b] : 0;
    const int S = a.sinks ? a.sinks[b] : 0;
    const float cap = a.softcap ? a.softcap[b] : 0.0f;
    // Non-causal rows see keys [0, ctx): plan and mask as if every row sat at
    // the last position.
    const bool causal = !MODS || a.mods.causal;
    const SplitPlan plan = causal ? plan_splits(cr.pos_min, cr.pos_max, W, S, a.split_tokens)
                                  : plan_splits(ctx - 1, ctx - 1, 0, 0, a.split_tokens);
    if (split >= plan.n_splits) {
        // Without a merge, the rows of a chunk that sees no key are written
        // here (once, by split 0).
        if (a.max_splits == 1 && plan.n_splits == 0) {
            for (int idx = tid; idx < (cr.r1 - cr.r0) * D; idx += 256) {
                const int rr = cr.r0 + idx / D;
                const int h = a.groups.list[gstart + rr % gsize];
                write_single_split(a, ((int64_t)b * a.q_len + rr / gsize) * a.hq + h, idx % D, -INFINITY, 0.0f, 0.0f);
            }
        }
        return;
    }
    int ka, kb;
    split_range(plan, split, a.split_tokens, &ka, &kb);

    // Stage the split's physical page ids (clamped into the arena).
    const int ps = a.page_shift;
    const int pmask = (1 << ps) - 1;
    const int p0 = ka >> ps;
    const int np = ((kb - 1) >> ps) - p0 + 1;
    for (int t = tid; t < np; t += 256) {
        int pid = a.page_table[(int64_t)b * a.max_pages + p0 + t];
        s_pid[t] = (REGEN && pid == -1) ? -1 : (((unsigned)pid < (unsigned)a.num_phys) ? pid : 0);
    }

    // Query slices and positions of the chunk's rows (MODS: also the bound
    // of the visible keys, the ALiBi slope and the mask row).
    float q[MC][DPL];
    int pos[MC];
    int posv[MC];
    float slope[MC];
    const uint32_t *mrow[MC];
#pragma unroll
    for (int r = 0; r < MC; ++r) {
        const int rr = cr.r0 + r;
        posv[r] = -1;
        slope[r] = 0.0f;
        mrow[r] = nullptr;
        if (rr < cr.r1) {
            const int i = rr / gsize;
            const int h = a.groups.list[gstart + rr % gsize];
            pos[r] = ctx - a.q_len + i;
            if constexpr (MODS) {
                posv[r] = causal ? pos[r] : ctx - 1;
                slope[r] = a.mods.alibi ? a.mods.alibi[h] : 0.0f;
                if (a.mods.mask)
                    mrow[r] = a.mods.mask + ((int64_t)b * a.q_len + i) * a.mods.mask_words;
            }
            const E *qrow = reinterpret_cast<const E *>(a.q) +
                            (((int64_t)b * a.q_len + i) * a.hq + h) * D;
#pragma unroll
            for (int n = 0; n < NL; ++n) {
                uint4 c = *reinterpret_cast<const uint4 *>(qrow + n * R * EPC + li * EPC);
                Elem<E>::unpack(c, &q[r][n * EPC]);
            }
        } else {
            pos[r] = -1;
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                q[r][e] = 0.0f;
        }
    }
    __syncthreads();

    float m[MC], l[MC], acc[MC][DPL];
#pragma unroll
    for (int r = 0; r < MC; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.0f;
#pragma unroll
        for (int e = 0; e < DPL; ++e)
            acc[r][e] = 0.0f;
    }

    const float qk_scale = a.scale;
    // REGEN: this sequence's generator key.
    uint32_t seq_key = (uint32_t)b;
    if constexpr (REGEN) {
        if (a.seq_keys) {
            const int sk = a.seq_keys[b];
            seq_key = (uint32_t)(sk < 0 ? 0 : (sk > 65535 ? 65535 : sk));
        }
    }
    const E *kbase = reinterpret_cast<const E *>(a.k_pages);
    const E *vbase = reinterpret_cast<const E *>(a.v_pages);
    const int64_t head_off = (int64_t)g << ps;  // rows before head g inside a page

    // Two register buffers in ping-pong: the next keys' loads are in flight
    // while the current ones are folded.  The prefetch is unconditional: past
    // the span the key index is clamped to the span's last row (cache hits,
    // no extra HBM traffic); a conditional load would make the compiler wait
    // for all loads where the branches join.
    struct Buf {
        uint4 k[KU][NL];
        uint4 v[KU][NL];
        uint32_t cold;  // REGEN: bit u set when key u's page is regenerated here
    };
    auto load = [&](Buf &bf, int base) {
        bf.cold = 0;
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int key = base + u * (4 * GPW) + wave * GPW + grp;
            const int jj = key < kb ? key : kb - 1;
            const int pid = s_pid[(jj >> ps) - p0];
            int64_t row = ((int64_t)pid * a.hkv << ps) + head_off + (jj & pmask);
            if constexpr (REGEN) {
                // A cold key's placeholder load reads row 0 of page 0.
                bf.cold |= (pid < 0 ? 1u : 0u) << u;
                row = pid < 0 ? head_off : row;
            }
            const E *kr = kbase + row * D;
            const E *vr = vbase + row * D;
#pragma unroll
            for (int n = 0; n < NL; ++n) {
                if constexpr (NT) {
                    bf.k[u][n] = stream_load16(kr + n * R * EPC + li * EPC);
                    bf.v[u][n] = stream_load16(vr + n * R * EPC + li * EPC);
                } else {
                    bf.k[u][n] = load16(kr + n * R * EPC + li * EPC);
                    bf.v[u][n] = load16(vr + n * R * EPC + li * EPC);
                }
            }
        }
    };
    // FULL: every key of the iteration is inside the span and at or before
    // every row's position, with no window: no per-key visibility test.
    // No floating-point contraction here: the FULL copy must round exactly
    // as the masked one (and as the generator instances) do, so that a key
    // folds to the same bits whichever copy or instance folds it.
    auto fold = [&](const Buf &bf, int base, auto full_tag) {
#pragma clang fp contract(off)
        constexpr bool FULL = decltype(full_tag)::value;
        float kv[KU][DPL], vv[KU][DPL];
        int key[KU];
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            key[u] = base + u * (4 * GPW) + wave * GPW + grp;
#pragma unroll
            for (int n = 0; n < NL; ++n) {
                Elem<E>::unpack(bf.k[u][n], &kv[u][n * EPC]);
                Elem<E>::unpack(bf.v[u][n], &vv[u][n * EPC]);
            }
        }
        if constexpr (REGEN) {
            static_assert(EPC == 4, "one generator call per 16-byte fp32 piece");
            if (bf.cold) {
#pragma unroll
                for (int u = 0; u < KU; ++u) {
                    if ((bf.cold >> u) & 1u) {
                        const uint32_t tok = (uint32_t)(key[u] < kb ? key[u] : kb - 1);
#pragma unroll
                        for (int n = 0; n < NL; ++n) {
                            const uint32_t quad = (uint32_t)(n * R + li);
                            regen_quad(a.regen_seed, (uint32_t)a.regen_layer, seq_key, 1u, (uint32_t)g, tok,
                                       quad, &kv[u][n * EPC]);
                            regen_quad(a.regen_seed, (uint32_t)a.regen_layer, seq_key, 2u, (uint32_t)g, tok,
                                       quad, &vv[u][n * EPC]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < MC; ++r) {
            float s2[KU];
#pragma unroll
            for (int u = 0; u < KU; ++u) {
                float part = 0.0f;
#pragma unroll
                for (int e = 0; e < DPL; ++e)
                    part = fmaf(q[r][e], kv[u][e], part);
                float s = group_sum<R>(part) * qk_scale;
                if (cap > 0.0f)
                    s = cap * tanhf(s / cap);
                const int j = key[u];
                bool vis;
                if constexpr (FULL) {
                    vis = true;
                } else if constexpr (MODS) {
                    s -= slope[r] * fabsf((float)(pos[r] - j));
                    vis = j < kb && j <= posv[r] && (W <= 0 || j > pos[r] - W || j < S);
                    if (mrow[r]) {
                        const int jm = j < kb ? j : kb - 1;  // in-bounds word
                        vis = vis && ((mrow[r][jm >> 5] >> (jm & 31)) & 1u);
                    }
                } else {
                    vis = j < kb && j <= pos[r] && (W <= 0 || j > pos[r] - W || j < S);
                }
                s2[u] = vis ? s * kLog2e : -INFINITY;
            }
            float mx = s2[0];
#pragma unroll
            for (int u = 1; u < KU; ++u)
                mx = fmaxf(mx, s2[u]);
            const float mnew = fmaxf(m[r], mx);
            const float msafe = mnew == -INFINITY ? 0.0f : mnew;
            const float alpha = fast_exp2(m[r] - msafe);
            float p[KU];
            float psum = 0.0f;
#pragma unroll
            for (int u = 0; u < KU; ++u) {
                p[u] = fast_exp2(s2[u] - msafe);
                psum += p[u];
            }
            l[r] = fmaf(l[r], alpha, psum);
#pragma unroll
            for (int e = 0; e < DPL; ++e) {
                float x = acc[r][e] * alpha;
#pragma unroll
                for (int u = 0; u < KU; ++u)
                    x = fmaf(p[u], vv[u][e], x);
                acc[r][e] = x;
            }
            m[r] = mnew;
        }
    };

    // Iterations ending at or before full_end see every key for every row
    // (plain instances with 2 to 32 / DPL rows only: elsewhere a second copy
    // of the loop body costs registers, i.e. occupancy or spills).
    const int full_end = W <= 0 ? (kb < cr.pos_min + 1 ? kb : cr.pos_min + 1) : -1;
    auto fold_any = [&](const Buf &bf, int base) {
        if constexpr (!REGEN && !MODS && MC >= 2 && MC * DPL <= 32) {
            if (base + KPI <= full_end) {
                fold(bf, base, std::true_type{});
                return;
            }
        }
        fold(bf, base, std::false_type{});
    };
    Buf ba, bb;
    int base = ka;
    load(ba, base);
    while (base < kb) {
        load(bb, base + KPI);
        fold_any(ba, base);
        base += KPI;
        if (base >= kb)
            break;
        load(ba, base + KPI);
        fold_any(bb, base);
        base += KPI;
    }

    // Combine the row groups of each wave (butterfly over lane offsets R..32).
#pragma unroll
    for (int off = R; off < 64; off <<= 1) {
#pragma unroll
        for (int r = 0; r < MC; ++r) {
            const float mo = __shfl_xor(m[r], off);
            const float lo = __shfl_xor(l[r], off);
            const float mnew = fmaxf(m[r], mo);
            const float msafe = mnew == -INFINITY ? 0.0f : mnew;
            const float a1 = fast_exp2(m[r] - msafe);
            const float a2 = fast_exp2(mo - msafe);
            l[r] = l[r] * a1 + lo * a2;
#pragma unroll
            for (int e = 0; e < DPL; ++e) {
                const float ao = __shfl_xor(acc[r][e], off);
                acc[r][e] = acc[r][e] * a1 + ao * a2;
            }
            m[r] = mnew;
        }
    }
    if (lane < R) {
#pragma unroll
        for (int r = 0; r < MC; ++r) {
            if (lane == 0) {
                s_m[wave][r] = m[r];
                s_l[wave][r] = l[r];
            }
#pragma unroll
            for (int n = 0; n < NL; ++n)
#pragma unroll
                for (int e = 0; e < EPC; ++e)
                    s_acc[wave][r][n * R * EPC + li * EPC + e] = acc[r][n * EPC + e];
        }
    }
    __syncthreads();

    // Combine the 4 waves and write this split's partial state per row (or,
    // with one split per row, the row's output and lse).
    for (int idx = tid; idx < MC * D; idx += 256) {
        const int r = idx / D;
        const int d = idx - r * D;
        const int rr = cr.r0 + r;
        if (rr >= cr.r1)
            continue;
        float mm = s_m[0][r];
#pragma unroll
        for (int w = 1; w < 4; ++w)
            mm = fmaxf(mm, s_m[w][r]);
        const float msafe = mm == -INFINITY ? 0.0f : mm;
        float ls = 0.0f, as = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float f = fast_exp2(s_m[w][r] - msafe);
            ls = fmaf(s_l[w][r], f, ls);
            as = fmaf(s_acc[w][r][d], f, as);
        }
        const int i = rr / gsize;
        const int h = a.groups.list[gstart + rr % gsize];
        const int64_t row_id = ((int64_t)b * a.q_len + i) * a.hq + h;
        if (a.max_splits == 1) {
            write_single_split(a, row_id, d, mm, ls, as);
            continue;
        }
        const int64_t slot = row_id * a.max_splits + split;
        a.ws_acc[slot * D + d] = as;
        if (d == 0) {
            a.ws_ml[slot * 2 + 0] = mm;
            a.ws_ml[slot * 2 + 1] = ls;
        }
    }
}

template <typename E, int D, int MC>
hipError_t launch_one(const SplitArgs &a, hipStream_t stream)
{
    // Keys per row group per step, sized so that two register buffers, the
    // query slices and the accumulators fit without spilling.
    constexpr int DPL = D / 16;
    constexpr int KU = (D == 64) ? ((MC <= 2) ? 8 : (MC * DPL <= 16 ? 4 : 2)) : ((MC <= 2) ? 4 : 2);
    dim3 grid(a.max_splits, a.hkv * a.n_chunks, a.batch);
    if (a.regen)
        hipLaunchKernelGGL((split_valu_kernel<E, D, MC, KU, true, false, false>), grid, dim3(256), 0, stream, a);
    else if (a.mods.any)
        hipLaunchKernelGGL((split_valu_kernel<E, D, MC, KU, false, true, false>), grid, dim3(256), 0, stream, a);
    else if (a.n_chunks == 1)
        hipLaunchKernelGGL((split_valu_kernel<E, D, MC, KU, false, false, true>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((split_valu_kernel<E, D, MC, KU, false, false, false>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_rows(const SplitArgs &a, hipStream_t stream)
{
    switch (a.rows_per_item) {
    case 1: return launch_one<E, D, 1>(a, stream);
    case 2: return launch_one<E, D, 2>(a, stream);
    case 4: return launch_one<E, D, 4>(a, stream);
    case 8: return launch_one<E, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_split_valu(const SplitArgs &a, hipStream_t stream)
{
    return a.head_dim == 64 ? launch_rows<float, 64>(a, stream) : launch_rows<float, 128>(a, stream);
}

}  // namespace atlas

// split_mfma.hip -- split-KV fold on the matrix cores (bf16 K/V).
//
// Same work items and partial states as split_valu.hip (one workgroup per
// (sequence, K/V head, chunk of rows, span of keys); plan.h fixes the spans),
// for bf16 inputs, where the vector ALUs alone cannot keep up with HBM: a
// group of 8 q-heads costs 4 flop per K/V byte.
//
// Per wave, 32 keys at a time (the 4 waves interleave 32-key chunks):
//   S^T = K Q^T     v_mfma_f32_16x16x32_bf16, A = 16 keys x 32 dims read
//                   from the wave's LDS K tile in the A-operand layout (each
//                   lane 16 contiguous bytes of one key row), B = Q^T for the
//                   item's <= 16 rows (q-heads of the group x queries) kept in
//                   registers; each lane ends up with 8 scores of one row.
//   softmax         row max over the 4 lanes that share a row (two xor
//                   shuffles), exp2 with the scale folded by log2(e), and a
//                   lazily rescaled accumulator (the reference max may lag the
//                   running max by up to 2^8; every term uses the same
//                   reference, so only rounding changes).
//   O^T += V^T P^T  v_mfma_f32_16x16x32_bf16 twice: P is split into a bf16
//                   high part and a bf16 remainder (together ~16 significant
//                   bits), so V stays exact bf16 with no range restriction.
//                   V is staged in the wave's own LDS tile and read transposed
//                   with ds_read_b64_tr_b16 (4 consecutive keys of one dim per
//                   read).
// The next chunk's K and V are loaded into registers as soon as the current
// chunk's have been consumed, so they are in flight during its softmax and
// P.V products.  K and V are both loaded as whole rows (1 KiB contiguous per
// wave instruction) and staged through the wave's LDS tiles; the loads are
// non-temporal (NT instances) when one row chunk holds every row of a K/V
// head, so that each row is read once per pass (several chunks re-read the
// same rows, which ordinary loads keep in cache).  Loaded straight into the
// A-operand layout, each K instruction read half of 16 cache lines (whose
// other halves the next instruction wanted from cache), which ruled out
// non-temporal loads for K there.
// At the end the 4 waves' states are combined in LDS and one (m, l, acc)
// partial per row is written; merge.hip finishes (with one split per row,
// the fold writes the output and lse itself, merge_row.h).
//
// fp32 queries over the bf16 cache (QF32 instances): each query element is
// carried as a bf16 high part and a bf16 remainder (~16 significant bits
// together), and S^T takes one product per part; K stays exact bf16.
//
// In-kernel regeneration (REGEN instances, atlas_attend_decode_regen):
// page-table entries of -1 mark pages that are not stored; a lane whose
// 16-byte piece (8 dims of one key row) falls in such a page builds it from
// the page regenerator's generator (philox.h: two calls of 4 dims each for K
// and for V, rounded to bf16 as the regenerator stores them) while the chunk
// is staged, so the fold sees the bits a regenerated page would hold.  Its
// placeholder load reads row 0 of page 0 of the K/V head, which stays cached.
#include "device.h"
#include "kernels.h"
#include "merge_row.h"
#include "philox.h"

namespace atlas {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kChunk = 32;            // keys per wave step
constexpr int kRowsMax = 16;          // rows per work item (MFMA N)
constexpr float kRescaleSlack = 8.0f;

template <int D>
struct alignas(16) SplitSmem {
    static constexpr int RS = D + 16; // padded LDS row (elements): 32-byte skew between rows
    static constexpr int RSK = D + 8; // K rows: 16-byte skew (conflict-free operand reads)
    union alignas(16) {
        uint16_t v[4][kChunk][RS];    // per-wave V tile (bf16 bits)
        float acc[4][kRowsMax][D];    // end-of-span wave states
    } u;
    alignas(16) uint16_t k[4][kChunk][RSK];  // per-wave K tile (bf16 bits)
    float m[4][kRowsMax];
    float l[4][kRowsMax];
    int32_t pid[kMaxSplitPages];
};

// bf16 pair (hi part, remainder) of two fp32 values, packed per part.
__device__ __forceinline__ void split_hi_lo(float p0, float p1, uint32_t &hi, uint32_t &lo)
{
    const bf16x2 h = __builtin_convertvector(f32x2{p0, p1}, bf16x2);
    hi = __builtin_bit_cast(uint32_t, h);
    const float r0 = p0 - bf16_lo(hi);
    const float r1 = p1 - bf16_hi(hi);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
}

// bf16 high parts and bf16 remainders of 8 fp32 values.
__device__ __forceinline__ void split_hi_lo8(const float *x, bf16x8 &hi, bf16x8 &lo)
{
    u32x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        uint32_t hh, ll;
        split_hi_lo(x[2 * e], x[2 * e + 1], hh, ll);
        h[e] = hh;
        l[e] = ll;
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// MODS instances (atlas_attend_mods): non-causal rows plan and mask over
// [0, ctx); ALiBi slopes and mask bits per (row, key).
template <int D, bool MODS, bool NT, bool QF32, bool REGEN>
__global__ __launch_bounds__(256) void split_mfma_kernel(SplitArgs a)
{
    constexpr int KS = D / 32;                 // QK k-steps
    constexpr int DT = D / 16;                 // output dim tiles
    constexpr int CPR = D / 8;                 // 16-byte pieces per row
    constexpr int VCH = kChunk * CPR / 64;     // V pieces per lane per chunk
    __shared__ SplitSmem<D> sm;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l16 = lane & 15;
    const int g4 = lane >> 4;

    const int split = blockIdx.x;
    const int g = blockIdx.y / a.n_chunks;
    const int chunk = blockIdx.y - g * a.n_chunks;
    const int b = blockIdx.z;
    const int gstart = a.groups.start[g];
    const int gsize = a.groups.start[g + 1] - gstart;

    int ctx = a.context_lens[b];
    ctx = ctx < 0 ? 0 : (ctx > a.max_context ? a.max_context : ctx);
    const ChunkRows cr = chunk_rows(chunk, kRowsMax, gsize, a.q_len, ctx);
    if (cr.r0 >= cr.r1)
        return;
    const int W = a.window ? a.window[b] : 0;
    const int S = a.sinks ? a.sinks[b] : 0;
    const float cap = a.softcap ? a.softcap[b] : 0.0f;
    const bool causal = !MODS || a.mods.causal;
    const SplitPlan plan = causal ? plan_splits(cr.pos_min, cr.pos_max, W, S, a.split_tokens)
                                  : plan_splits(ctx - 1, ctx - 1, 0, 0, a.split_tokens);
    if (split >= plan.n_splits) {
        // Without a merge, the rows of a chunk that sees no key are written
        // here (once, by split 0).
        if (a.max_splits == 1 && plan.n_splits == 0) {
            for (int idx = tid; idx < (cr.r1 - cr.r0) * D; idx += 256) {
                const int row = cr.r0 + idx / D;
                const int hh = a.groups.list[gstart + row % gsize];
                write_single_split(a, ((int64_t)b * a.q_len + row / gsize) * a.hq + hh, idx % D, -INFINITY, 0.0f,
                                   0.0f);
            }
        }
        return;
    }
    int ka, kb;
    split_range(plan, split, a.split_tokens, &ka, &kb);

    const int ps = a.page_shift;
    const int pmask = (1 << ps) - 1;
    const int p0 = ka >> ps;
    const int np = ((kb - 1) >> ps) - p0 + 1;
    for (int t = tid; t < np; t += 256) {
        int pid = a.page_table[(int64_t)b * a.max_pages + p0 + t];
        sm.pid[t] = (REGEN && pid == -1) ? -1 : (((unsigned)pid < (unsigned)a.num_phys) ? pid : 0);
    }
    // REGEN: this sequence's generator key.
    uint32_t seq_key = (uint32_t)b;
    if constexpr (REGEN) {
        if (a.seq_keys) {
            const int sk = a.seq_keys[b];
            seq_key = (uint32_t)(sk < 0 ? 0 : (sk > 65535 ? 65535 : sk));
        }
    }

    // This lane's row (column of the S^T / O^T tiles) and its query operand.
    const int rr = cr.r0 + l16;
    const bool row_ok = rr < cr.r1;
    const int qi = row_ok ? rr / gsize : 0;
    const int h = row_ok ? a.groups.list[gstart + rr % gsize] : 0;
    const int pos = row_ok ? ctx - a.q_len + qi : -1;
    // MODS: bound of the visible keys, ALiBi slope and mask row of this row.
    const int posv = (MODS && !causal && row_ok) ? ctx - 1 : pos;
    const float slope = (MODS && row_ok && a.mods.alibi) ? a.mods.alibi[h] : 0.0f;
    const uint32_t *mrow =
        (MODS && row_ok && a.mods.mask) ? a.mods.mask + ((int64_t)b * a.q_len + qi) * a.mods.mask_words : nullptr;
    bf16x8 qf[KS];
    bf16x8 qlo[QF32 ? KS : 1];  // QF32: the remainders of the query
    {
        const int64_t qoff = (((int64_t)b * a.q_len + qi) * a.hq + h) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if constexpr (QF32) {
                float x[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
                if (row_ok) {
                    const float *qrow = reinterpret_cast<const float *>(a.q) + qoff + 32 * s + 8 * g4;
                    const f32x4 x0 = *reinterpret_cast<const f32x4 *>(qrow);
                    const f32x4 x1 = *reinterpret_cast<const f32x4 *>(qrow + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[e] = x0[e];
                        x[4 + e] = x1[e];
                    }
                }
                split_hi_lo8(x, qf[s], qlo[s]);
            } else {
                const uint16_t *qrow = reinterpret_cast<const uint16_t *>(a.q) + qoff;
                qf[s] = row_ok ? *reinterpret_cast<const bf16x8 *>(qrow + 32 * s + 8 * g4) : bf16x8{};
            }
        }
    }
    __syncthreads();

    const uint16_t *kpages = reinterpret_cast<const uint16_t *>(a.k_pages);
    const uint16_t *vpages = reinterpret_cast<const uint16_t *>(a.v_pages);
    const int64_t head_rows = (int64_t)g << ps;
    // Register buffer for one chunk's K and V, both staged through LDS: each
    // wave instruction reads whole rows (1 KiB runs).
    struct Regs {
        uint4 k[VCH];
        uint4 v[VCH];
        uint32_t cold;  // REGEN: bit u set when piece u's page is regenerated here
    };
    auto load_chunk = [&](Regs &r, int cb) {
        r.cold = 0;
#pragma unroll
        for (int u = 0; u < VCH; ++u) {
            const int c = lane + 64 * u;
            const int key = c / CPR;
            const int col = c - key * CPR;
            // Key row (clamped to the span's last key).
            const int j = cb + key;
            const int jj = j < kb ? j : kb - 1;
            const int pid = sm.pid[(jj >> ps) - p0];
            int64_t row = (((int64_t)pid * a.hkv) << ps) + head_rows + (jj & pmask);
            if constexpr (REGEN) {
                // A cold key's placeholder load reads row 0 of page 0.
                r.cold |= (pid < 0 ? 1u : 0u) << u;
                row = pid < 0 ? head_rows : row;
            }
            const int64_t off = row * D + col * 8;
            if constexpr (NT) {
                r.k[u] = stream_load16(kpages + off);
                r.v[u] = stream_load16(vpages + off);
            } else {
                r.k[u] = load16(kpages + off);
                r.v[u] = load16(vpages + off);
            }
        }
    };

    const float qk_scale = a.scale;
    float m_ref = -INFINITY;
    float l_part = 0.0f;
    f32x4 acc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
        acc[t] = f32x4{};

    // One chunk: V into the wave's LDS tile and S^T from the registers, then
    // (once both are consumed) the next chunk's loads into the same
    // registers, then softmax and O^T += V^T P^T from LDS.
    auto fold_chunk = [&](Regs &r, int cb, int cb_next) {
        // REGEN: the pieces of cold keys come from the generator.
        if constexpr (REGEN) {
            if (r.cold) {
#pragma unroll
                for (int u = 0; u < VCH; ++u) {
                    if ((r.cold >> u) & 1u) {
                        const int c = lane + 64 * u;
                        const int key = c / CPR;
                        const int col = c - key * CPR;
                        const uint32_t tok = (uint32_t)(cb + key < kb ? cb + key : kb - 1);
                        uint32_t w[2][4];
#pragma unroll
                        for (int t = 0; t < 2; ++t) {
#pragma unroll
                            for (int hq4 = 0; hq4 < 2; ++hq4) {
                                float z[4];
                                regen_quad(a.regen_seed, (uint32_t)a.regen_layer, seq_key, 1u + t, (uint32_t)g,
                                           tok, (uint32_t)(2 * col + hq4), z);
                                w[t][2 * hq4 + 0] = f32_to_bf16_bits(z[0]) | (f32_to_bf16_bits(z[1]) << 16);
                                w[t][2 * hq4 + 1] = f32_to_bf16_bits(z[2]) | (f32_to_bf16_bits(z[3]) << 16);
                            }
                        }
                        r.k[u] = make_uint4(w[0][0], w[0][1], w[0][2], w[0][3]);
                        r.v[u] = make_uint4(w[1][0], w[1][1], w[1][2], w[1][3]);
                    }
                }
            }
        }
        // Stage this chunk's K and V in the wave's LDS tiles, then refill
        // the registers with the next chunk.
#pragma unroll
        for (int u = 0; u < VCH; ++u) {
            const int c = lane + 64 * u;
            const int key = c / CPR;
            const int col = c - key * CPR;
            *reinterpret_cast<uint4 *>(&sm.k[wave][key][col * 8]) = r.k[u];
            *reinterpret_cast<uint4 *>(&sm.u.v[wave][key][col * 8]) = r.v[u];
        }
        load_chunk(r, cb_next);
        // The tiles' reads must follow their writes in this wave.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // S^T tiles: lane holds row l16, keys 16t + 4*g4 + j.  The two tiles'
        // chains alternate.
        f32x4 st[2] = {f32x4{}, f32x4{}};
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(&sm.k[wave][16 * t + l16][32 * s + 8 * g4]);
                st[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], st[t], 0, 0, 0);
                if constexpr (QF32)
                    st[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qlo[s], st[t], 0, 0, 0);
            }

        // Scale, softcap, mask (log2 units).
        float x[8];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int key = cb + 16 * t + 4 * g4 + j;
                float sc = st[t][j] * qk_scale;
                if (cap > 0.0f)
                    sc = cap * tanhf(sc / cap);
                bool vis;
                if constexpr (MODS) {
                    sc -= slope * fabsf((float)(pos - key));
                    vis = key < kb && key <= posv && (W <= 0 || key > pos - W || key < S);
                    if (mrow) {
                        const int km = key < kb ? key : kb - 1;  // in-bounds word
                        vis = vis && ((mrow[km >> 5] >> (km & 31)) & 1u);
                    }
                } else {
                    vis = key < kb && key <= pos && (W <= 0 || key > pos - W || key < S);
                }
                x[4 * t + j] = vis ? sc * kLog2e : -INFINITY;
            }
        float mx = x[0];
#pragma unroll
        for (int e = 1; e < 8; ++e)
            mx = fmaxf(mx, x[e]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (mx > m_ref + kRescaleSlack) {
            const float alpha = fast_exp2(m_ref - mx);
            l_part *= alpha;
#pragma unroll
            for (int t = 0; t < DT; ++t)
                acc[t] *= alpha;
            m_ref = mx;
        }
        const float msafe = m_ref == -INFINITY ? 0.0f : m_ref;
        u32x4 phi, plo;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const float p0v = fast_exp2(x[e] - msafe);
            const float p1v = fast_exp2(x[e + 1] - msafe);
            l_part += p0v + p1v;
            uint32_t hi, lo;
            split_hi_lo(p0v, p1v, hi, lo);
            phi[e >> 1] = hi;
            plo[e >> 1] = lo;
        }
        const bf16x8 pbh = __builtin_bit_cast(bf16x8, phi);
        const bf16x8 pbl = __builtin_bit_cast(bf16x8, plo);

        // O^T += V^T P^T: slots 0..3 = keys 4*g4 + k, slots 4..7 = 16 + 4*g4 + k.
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int key0 = 4 * g4 + (l16 >> 2);
            const int dim0 = 16 * dt + 4 * (l16 & 3);
            const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(&sm.u.v[wave][key0][dim0]));
            const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(&sm.u.v[wave][key0 + 16][dim0]));
            // Whole-vector concatenation (element-wise extraction from these
            // reads is mis-compiled by this toolchain).
            const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pbh, acc[dt], 0, 0, 0);
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pbl, acc[dt], 0, 0, 0);
        }
        // The next chunk's writes must not overtake these reads.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // The prefetch is unconditional: past the span every address is clamped
    // to the span's last row (cache hits, no extra HBM traffic), and a
    // conditional load would make the compiler wait for all loads at the join.
    // One register buffer: its next contents are loaded as soon as the
    // current ones are consumed, so the loads are in flight during the
    // softmax and the P.V products (and two waves fit per SIMD).
    constexpr int kStride = 4 * kChunk;  // the 4 waves interleave chunks
    Regs rg;
    int cb = ka + kChunk * wave;
    if (cb < kb)
        load_chunk(rg, cb);
    for (; cb < kb; cb += kStride)
        fold_chunk(rg, cb, cb + kStride);

    // Per-row sum of the four lane groups.
    l_part += __shfl_xor(l_part, 16);
    l_part += __shfl_xor(l_part, 32);
    __syncthreads();  // every wave is done with its V tile (the state area aliases it)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            sm.u.acc[wave][l16][16 * dt + 4 * g4 + j] = acc[dt][j];
    if (g4 == 0) {
        sm.m[wave][l16] = m_ref;
        sm.l[wave][l16] = l_part;
    }
    __syncthreads();

    for (int idx = tid; idx < kRowsMax * D; idx += 256) {
        const int r = idx / D;
        const int d = idx - r * D;
        const int row = cr.r0 + r;
        if (row >= cr.r1)
            continue;
        float mm = sm.m[0][r];
#pragma unroll
        for (int w = 1; w < 4; ++w)
            mm = fmaxf(mm, sm.m[w][r]);
        const float msafe = mm == -INFINITY ? 0.0f : mm;
        float ls = 0.0f, as = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float f = fast_exp2(sm.m[w][r] - msafe);
            ls = fmaf(sm.l[w][r], f, ls);
            as = fmaf(sm.u.acc[w][r][d], f, as);
        }
        const int i = row / gsize;
        const int hh = a.groups.list[gstart + row % gsize];
        if (a.max_splits == 1) {
            write_single_split(a, ((int64_t)b * a.q_len + i) * a.hq + hh, d, mm, ls, as);
            continue;
        }
        const int64_t slot = (((int64_t)b * a.q_len + i) * a.hq + hh) * a.max_splits + split;
        a.ws_acc[slot * D + d] = as;
        if (d == 0) {
            a.ws_ml[slot * 2 + 0] = mm;
            a.ws_ml[slot * 2 + 1] = ls;
        }
    }
}

template <int D, bool QF32>
void (*pick_split_mfma(const SplitArgs &a))(SplitArgs)
{
    if (a.regen)
        return split_mfma_kernel<D, false, false, QF32, true>;
    if (a.mods.any)
        return split_mfma_kernel<D, true, false, QF32, false>;
    return a.n_chunks == 1 ? split_mfma_kernel<D, false, true, QF32, false> : split_mfma_kernel<D, false, false, QF32, false>;
}

}  // namespace

hipError_t launch_split_mfma(const SplitArgs &a, hipStream_t stream)
{
    if (a.rows_per_item != kRowsMax || (a.regen && a.mods.any))
        return hipErrorInvalidValue;
    dim3 grid(a.max_splits, a.hkv * a.n_chunks, a.batch);
    void (*kernel)(SplitArgs);
    if (a.head_dim == 64)
        kernel = a.q_f32 ? pick_split_mfma<64, true>(a) : pick_split_mfma<64, false>(a);
    else
        kernel = a.q_f32 ? pick_split_mfma<128, true>(a) : pick_split_mfma<128, false>(a);
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace atlas

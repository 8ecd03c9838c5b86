// prefill_mfma.hip -- tiled causal prefill on the gfx950 matrix cores (bf16).
//
// CPUAttn README: the parallel lowering runs a fused QK -> Mod/RowNorm -> PV
// tile pipeline, and an exact causal mask stops each query block at the last
// key block it can reach.  This kernel is that pipeline for a paged bf16 K/V
// history, with the cache-backed suffix positions of the same page (query i
// of a sequence with L keys sits at position L - q_len + i):
//
//   workgroup  = 256 rows x one K/V head: the rows are (query position, q-head
//                of the group) pairs, so a K/V tile staged in LDS serves all
//                q-heads of the group (grouped-query attention);
//   key blocks = 64 keys; block kb runs only while kb*64 <= the last row's
//                position (causal block-stop); with a sliding window the
//                blocks before the lowest row's window start are skipped
//                (except the blocks holding the sink keys); only blocks some
//                row does not see whole apply the per-row mask; a softcap is
//                applied to the scores before the mask, each score carried
//                as -1/(1 + 2^(k s)) (ordered like the capped logit) with the
//                cap's affine map folded into the exponent's FMA;
//   per wave   = 32 rows.  S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K
//                from LDS, B = Q held in registers), so each lane owns one
//                row's scores and the row max is lane-local plus one swap
//                between the two lane halves; online softmax with exp2 and
//                the scale folded by log2(e); rescaling of the accumulator is
//                skipped while the running max grows by less than 2^8
//                (results are the same up to rounding: every term uses the
//                same reference max); P is rounded to fp16 (11-bit
//                mantissa), the row sum is taken over those fp16 values
//                (v_dot2_f32_f16), and O^T += V^T P^T runs on
//                v_mfma_f32_32x32x16_f16, with V converted bf16 -> fp16 while
//                it is staged and read transposed by ds_read_b64_tr_b16.
//                fp32 accumulation throughout, fp32 output.
//   pipeline   = the next key block is fetched into registers while the
//                current one is computed, then written to the other LDS
//                buffer: one barrier per block.
//   grid       = heavy-first: the query blocks with the most keys launch
//                first; consecutive workgroups cycle over K/V heads, so all
//                workgroups of one K/V head land on the same XCD (the
//                hardware deals workgroups to the 8 XCDs round-robin) and
//                share its L2.
//
// Modifications (MODS instances, atlas_attend_mods): non-causal rows take
// every key block of the context, with only the block past the last key
// masked.  Mask bits hide keys per (row, key): a pass over the workgroup's
// mask rows lists the key blocks some row sees and marks those every row
// sees whole, which skip the per-score mask bits; the others load each
// lane's two mask words one block ahead, with the block's K/V.  An ALiBi
// slope adds -slope |pos - j| (as -slope/scale |pos - j| in the units of the
// raw product, after the softcap): one FMA per score for the per-key part,
// the per-row part folded into the row max and the exponent's offset; the
// key blocks then run outward from the diagonal (leftwards, then rightwards
// for non-causal rows), so the first block holds nearly the row max and the
// accumulator is seldom rescaled.
//
// Precondition of the fp16 P.V product: |V| <= 65504 (validation mode
// checks it).  Scores use bf16 K and Q exactly (products are exact in fp32).
#include "device.h"
#include "kernels.h"

namespace atlas {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWaves = 8;
constexpr int kRows = 32 * kWaves;   // rows per workgroup
constexpr int kBN = 64;              // keys per block
constexpr int kPad = 24;             // LDS row padding (elements): conflict-free K rows, best transposed V reads
constexpr float kRescaleSlack = 8.0f;  // log2 units the running max may lag
constexpr int kPidWindow = 2048;       // page ids staged in LDS at a time
constexpr int kMaxListed = 4096;       // candidate key blocks a mask can thin out (longer: all computed)

// 16-byte alignment lets every K/V row piece move with one ds_read_b128 /
// ds_write_b128 (without it the compiler splits them into 4-byte pairs).
template <int D>
struct alignas(16) Smem {
    alignas(16) uint16_t k[2][kBN][D + kPad];  // bf16 bits
    alignas(16) uint16_t v[2][kBN][D + kPad];  // fp16 bits
    alignas(16) int32_t pid[kPidWindow];       // physical ids of pages [pid_base, pid_base + kPidWindow)
};

__device__ __forceinline__ uint32_t bf16pair_to_f16pair(uint32_t x)
{
    f32x2 f = {bf16_lo(x), bf16_hi(x)};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
}

// CAP: the call has per-sequence softcaps (plain instances only; the MODS
// instances take them at run time).  Without it no softcap code is compiled.
template <int D, bool MODS, bool CAP>
__global__ __launch_bounds__(512) void prefill_kernel(PrefillArgs a)
{
    constexpr int KS = D / 16;            // k-steps of the QK product
    constexpr int DT = D / 32;            // 32-dim tiles of the output
    constexpr int CPR = D / 8;            // 16-byte chunks per K/V row
    constexpr int CH = kBN * CPR / 512;   // chunks per thread per tile
    __shared__ Smem<D> sm;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int half = lane >> 5;

    // Heavy-first workgroup order; consecutive ids cycle over (b, K/V head).
    // Key splits (split_blocks > 0): consecutive workgroups of a query block
    // take consecutive runs of its key-block list.
    const int per_q = a.batch * a.hkv;
    const int qs = blockIdx.x / per_q;
    const int rem = blockIdx.x - qs * per_q;
    const int nspl = a.split_blocks > 0 ? a.max_splits : 1;
    const int qb_rev = qs / nspl;
    const int split = qs - qb_rev * nspl;
    const int b = rem / a.hkv;
    const int g = rem - b * a.hkv;
    const int qblock = a.n_qblocks - 1 - qb_rev;
    const int G = a.groups.max_group;
    const int npos = kRows / G;
    const int gstart = a.groups.start[g];
    const int gsize = a.groups.start[g + 1] - gstart;

    int ctx = a.context_lens[b];
    ctx = ctx < 0 ? 0 : (ctx > a.max_context ? a.max_context : ctx);
    const int i0 = qblock * npos;
    const int i1 = i0 + npos < a.q_len ? i0 + npos : a.q_len;
    const int pos_lo = ctx - a.q_len + i0;
    const int pos_hi = ctx - a.q_len + i1 - 1;
    // Per-sequence variants: sliding window of W keys (0 = off), the first S
    // keys always visible where a window is set, softcap cap (0 = off).
    const int W = a.window ? a.window[b] : 0;
    const int S = (a.sinks && W > 0) ? a.sinks[b] : 0;
    const float cap = ((MODS || CAP) && a.softcap) ? a.softcap[b] : 0.0f;
    // Last key any row of the block can see: the diagonal, or the whole
    // context for non-causal rows.
    const bool causal = !MODS || a.mods.causal;
    const int key_hi = causal ? pos_hi : (pos_hi >= 0 ? ctx - 1 : -1);

    // This lane's row.
    const int r = wave * 32 + (lane & 31);
    const int ri = r / G;
    const int rj = r - ri * G;
    const int qi = i0 + ri;
    const bool row_ok = ri < npos && qi < i1 && rj < gsize;
    const int pos = row_ok ? ctx - a.q_len + qi : -1;
    const int h = row_ok ? a.groups.list[gstart + rj] : 0;
    // MODS: this row's last visible key, ALiBi slope in raw-product units and
    // mask row.
    const int posv = causal ? pos : (row_ok ? ctx - 1 : -1);
    const float slope_raw = (MODS && row_ok && a.mods.alibi) ? a.mods.alibi[h] / a.scale : 0.0f;
    const uint32_t *mrow =
        (MODS && row_ok && a.mods.mask) ? a.mods.mask + ((int64_t)b * a.q_len + qi) * a.mods.mask_words : nullptr;
    // ALiBi on a key block starting at k0 is slope (k0 - pos) + slope jo over
    // its keys jo = j - k0 (both negated for a block at or right of the row):
    // one FMA with a constant per score for the per-key part, while the
    // per-lane part joins the row max and the exponent's offset.
    const bool alibi_on = MODS && a.mods.alibi != nullptr;

    bf16x8 qf[KS];
    {
        const uint16_t *qrow = reinterpret_cast<const uint16_t *>(a.q) +
                               (((int64_t)b * a.q_len + (row_ok ? qi : 0)) * a.hq + h) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            if (row_ok)
                qf[s] = *reinterpret_cast<const bf16x8 *>(qrow + 16 * s + 8 * half);
            else
                qf[s] = bf16x8{};
        }
    }

    const int ps = a.page_shift;
    const int pmask = (1 << ps) - 1;
    const uint16_t *kpages = reinterpret_cast<const uint16_t *>(a.k_pages);
    const uint16_t *vpages = reinterpret_cast<const uint16_t *>(a.v_pages);
    const int32_t *ptab = a.page_table + (int64_t)b * a.max_pages;

    // Page ids come from LDS, so a block's K/V loads never wait on a
    // page-table load.  Staged by windows of kPidWindow pages (one window
    // covers every page of all but extremely long, finely paged histories);
    // a window ends at the block's last page when the blocks run backwards.
    int pid_base = 0;
    auto stage_pids = [&](int first_page) {
        if (MODS && first_page < 0)
            first_page = 0;
        pid_base = first_page;
        const int last_page = key_hi >= 0 ? key_hi >> ps : -1;
        for (int t = tid; t < kPidWindow && first_page + t <= last_page; t += 512) {
            const int pid = ptab[first_page + t];
            sm.pid[t] = ((unsigned)pid < (unsigned)a.num_phys) ? pid : 0;
        }
    };

    // Global -> registers for key block kb (zeros past the last visible key).
    // Thread t stages CH adjacent 16-byte pieces of one row: one page lookup.
    const int srow = (tid * CH) / CPR;
    const int scol = (tid * CH) - srow * CPR;
    uint4 kreg[CH], vreg[CH];
    auto fetch = [&](int kb) {
        const int j = kb * kBN + srow;
        if (j <= key_hi) {
            const int pid = sm.pid[(j >> ps) - pid_base];
            const int64_t off = ((((int64_t)pid * a.hkv + g) << ps) + (j & pmask)) * D + scol * 8;
#pragma unroll
            for (int u = 0; u < CH; ++u) {
                kreg[u] = *reinterpret_cast<const uint4 *>(kpages + off + 8 * u);
                vreg[u] = *reinterpret_cast<const uint4 *>(vpages + off + 8 * u);
            }
        } else {
#pragma unroll
            for (int u = 0; u < CH; ++u) {
                kreg[u] = make_uint4(0, 0, 0, 0);
                vreg[u] = make_uint4(0, 0, 0, 0);
            }
        }
    };
    // Registers -> LDS buffer (V converted to fp16).
    auto stash = [&](int buf) {
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            const int row = srow;
            const int col = scol + u;
            *reinterpret_cast<uint4 *>(&sm.k[buf][row][col * 8]) = kreg[u];
            uint4 v16;
            v16.x = bf16pair_to_f16pair(vreg[u].x);
            v16.y = bf16pair_to_f16pair(vreg[u].y);
            v16.z = bf16pair_to_f16pair(vreg[u].z);
            v16.w = bf16pair_to_f16pair(vreg[u].w);
            *reinterpret_cast<uint4 *>(&sm.v[buf][row][col * 8]) = v16;
        }
    };

    const float c_log2 = a.scale * kLog2e;
    float m_ref = -INFINITY;  // reference max (log2 units) the accumulator is scaled to
    float l_part = 0.0f;      // this lane-half's share of the softmax denominator
    f32x16 acc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
        acc[t] = f32x16{};

    // Key blocks the rows can see: with a window, the sink blocks and then
    // the blocks from the lowest row's window start to the diagonal (blocks
    // in between are skipped); otherwise every block up to the diagonal.
    const TiledBlocks tbk = tiled_blocks(pos_lo, key_hi, W, S, kBN);
    int c_lo = 0, n_iter = tbk.n;
    if (a.split_blocks > 0) {
        // This workgroup's run of the list; past the query block's last run
        // there is nothing to do (uniform, before any barrier).
        c_lo = split * a.split_blocks;
        if (c_lo >= tbk.n)
            return;
        n_iter = c_lo + a.split_blocks < tbk.n ? a.split_blocks : tbk.n - c_lo;
    }
    auto block_at = [&](int it) { return tiled_block_at(tbk, c_lo + it); };

    // MODS with mask bits: the candidate blocks whose mask words are zero for
    // every row of this workgroup are dropped; the rest are listed in order
    // (wave 0 compacts the flags with a ballot), each marked full when every
    // row's 64 bits are set (its mask bits are then not applied per score).
    // The tests are conservative: a listed block may still be wholly hidden
    // by the causal or window rule.  Consecutive threads read consecutive
    // blocks of one mask row.
    __shared__ int32_t s_blk[MODS ? kMaxListed : 1];   // block * 2 + partial
    __shared__ uint8_t s_need[MODS ? kMaxListed : 1];
    __shared__ uint8_t s_part[MODS ? kMaxListed : 1];
    __shared__ int32_t s_count;
    __shared__ int32_t s_pivot;
    int n_run = n_iter;
    bool listed = false;
    // ALiBi: listed blocks whose first key is at or left of the last row's
    // position (the blocks run outward from the diagonal, see below).
    const int kb_diag = pos_hi >= 0 ? pos_hi / kBN : -1;
    int n_left = 0;
    if constexpr (MODS) {
        if (a.mods.mask && n_iter > 0 && n_iter <= kMaxListed) {
            listed = true;
            for (int i = tid; i < n_iter; i += 512) {
                s_need[i] = 0;
                s_part[i] = 0;
            }
            __syncthreads();
            const int rows_pos = i1 - i0;
            const int wl = a.mods.mask_words - 1;
            for (int idx = tid; idx < n_iter * rows_pos; idx += 512) {
                const int pp = idx / n_iter;
                const int c = idx - pp * n_iter;
                const uint32_t *m = a.mods.mask + ((int64_t)b * a.q_len + i0 + pp) * a.mods.mask_words;
                const int w = (block_at(c) * kBN) >> 5;
                const uint32_t m0 = m[w < wl ? w : wl];
                const uint32_t m1 = m[w + 1 < wl ? w + 1 : wl];
                if ((m0 | m1) != 0u)
                    s_need[c] = 1;
                if ((m0 & m1) != ~0u || w + 1 > wl)
                    s_part[c] = 1;
            }
            __syncthreads();
            if (wave == 0) {
                int base = 0, left = 0;
                for (int c0 = 0; c0 < n_iter; c0 += 64) {
                    const int c = c0 + lane;
                    const bool f = c < n_iter && s_need[c];
                    const uint64_t bal = __ballot(f);
                    if (f)
                        s_blk[base + __popcll(bal & ((1ull << lane) - 1ull))] = block_at(c) * 2 + s_part[c];
                    base += __popcll(bal);
                    left += __popcll(__ballot(f && block_at(c) <= kb_diag));
                }
                if (lane == 0) {
                    s_count = base;
                    s_pivot = left;
                }
            }
            __syncthreads();
            n_run = s_count;
            n_left = s_pivot;
        } else {
            // Entries of this run of the ascending list at or left of kb_diag.
            int le = kb_diag < 0 ? 0
                     : kb_diag < tbk.n_sink ? kb_diag + 1
                                            : tbk.n_sink + (kb_diag - tbk.first_win + 1);
            le = le < tbk.n_sink ? (kb_diag < tbk.n_sink ? le : tbk.n_sink) : (le > tbk.n ? tbk.n : le);
            le -= c_lo;
            n_left = le < 0 ? 0 : (le > n_iter ? n_iter : le);
        }
    }
    // Block order.  With ALiBi the bias falls with the distance from the
    // row, so the blocks run from the diagonal leftwards and then rightwards
    // (non-causal rows): the first block holds (nearly) the row max and the
    // accumulator is rarely rescaled; forward otherwise.
    const int d_last = alibi_on ? n_left - 1 : -1;
    auto list_at = [&](int it) { return (MODS && it <= d_last) ? d_last - it : it; };
    auto run_block = [&](int it) {
        const int i = list_at(it);
        return (MODS && listed) ? s_blk[i] >> 1 : block_at(i);
    };
    // First page to stage for block kb when the walk goes backwards from it.
    auto back_first = [&](int kbx) { return ((kbx * kBN + kBN - 1) >> ps) - kPidWindow + 1; };

    if (n_run > 0)
        stage_pids(d_last >= 0 ? back_first(run_block(0)) : (run_block(0) * kBN) >> ps);
    __syncthreads();  // page ids staged
    // MODS: the row's mask words for a block's two 32-key tiles (words past
    // the row's end hold keys beyond every context and are clamped); full
    // blocks need none.  Loaded one block ahead with the K/V, so the stash's
    // wait covers them and the next block reads them without waiting.
    auto is_partial = [&](int it) { return !(MODS && listed) || (s_blk[list_at(it)] & 1); };
    auto mask_words = [&](int it, int kbx, uint32_t &m0, uint32_t &m1) {
        if (mrow && is_partial(it)) {
            const int w = (kbx * kBN) >> 5;
            const int wl = a.mods.mask_words - 1;
            m0 = mrow[w < wl ? w : wl];
            m1 = mrow[w + 1 < wl ? w + 1 : wl];
        }
    };
    uint32_t mw0 = ~0u, mw1 = ~0u;  // the current block's mask words
    if (n_run > 0) {
        if constexpr (MODS)
            mask_words(0, run_block(0), mw0, mw1);
        fetch(run_block(0));
        stash(0);
    }
    // Complete the query loads here, once, after the page ids and the first
    // block's K/V were requested beside them: the asm "redefines" qf, so
    // inside the loop the compiler knows no load into qf is pending and does
    // not wait on the (prefetch) load counter before the first QK product.
#pragma unroll
    for (int s = 0; s < KS; ++s)
        asm volatile("" : "+v"(qf[s]));
    __syncthreads();

    for (int it = 0; it < n_run; ++it) {
        const int kb = run_block(it);
        const int cur = it & 1;
        const bool more = it + 1 < n_run;
        const int kb_next = more ? run_block(it + 1) : kb;
        if (more && ((((kb_next * kBN + kBN - 1) >> ps) - pid_base) >= kPidWindow ||
                     (MODS && ((kb_next * kBN) >> ps) < pid_base))) {
            // Uniform across the workgroup: move the page-id window.
            __syncthreads();
            stage_pids((MODS && kb_next < kb) ? back_first(kb_next) : (kb_next * kBN) >> ps);
            __syncthreads();
        }
        const int k0 = kb * kBN;
        const bool part = is_partial(it);
        uint32_t nw0 = ~0u, nw1 = ~0u;
        if constexpr (MODS) {
            if (more) {
                mask_words(it + 1, kb_next, nw0, nw1);
                fetch(kb_next);
            }
        } else {
            if (more)
                fetch(kb_next);
        }
        // S^T for the block: two 32-key tiles.
        f32x16 st[2] = {f32x16{}, f32x16{}};
        __builtin_amdgcn_s_setprio(1);
        // The two tiles' accumulation chains alternate: back-to-back
        // products into one accumulator would wait on each other.
#pragma unroll
        for (int s = 0; s < KS; ++s) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const bf16x8 kf =
                    *reinterpret_cast<const bf16x8 *>(&sm.k[cur][32 * t + (lane & 31)][16 * s + 8 * half]);
                st[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], st[t], 0, 0, 0);
            }
        }
        // Keep the K operand reads a few products ahead of their use.
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < 2 * KS - 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);

        __builtin_amdgcn_s_setprio(0);

        // Softcap (before the mask).  The capped logit cap tanh(s scale / cap)
        // is, in log2 units, L - 2L / (1 + 2^(k2 s)) with L = cap log2(e) and
        // k2 = 2 scale log2(e) / cap.  Each score becomes v = -1 / (1 + 2^(k2 s)),
        // which orders like the capped logit, so the mask and the row max
        // below apply unchanged and the map v -> 2L v + L replaces the scale
        // (lg_mul, lg_add).  With ALiBi, which is added after the cap in
        // raw-product units, the capped logit is formed in those units
        // instead.  The hardware exponential and reciprocal keep the logit
        // error under cap * 1e-6.
        float lg_mul = c_log2, lg_add = 0.0f;
        if (cap > 0.0f) {
            const float k2 = 2.0f * kLog2e * a.scale / cap;
            // Small scores (every |scale s / cap| <= 0.2 in this wave's
            // tiles, the usual case; CAP instances, whose registers allow
            // the third path): tanh(y) = y - y^3/3 + 2 y^5/15 with an error
            // below 17/315 y^7 <= 6.9e-7, so the capped logit in raw units is
            // s (1 + u (c1 + u c2)), u = s^2, c1 = -(scale/cap)^2/3,
            // c2 = 2 (scale/cap)^4/15: four full-rate operations in place of
            // the exponential and the reciprocal.
            bool small = false;
            const float rr = a.scale / cap;
            if constexpr (CAP) {
                float amax = 0.0f;
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        amax = fmaxf(amax, fabsf(st[t][e]));
                small = __all(amax <= 0.2f / rr);
            }
            if (small) {
                const float c1 = -(rr * rr) * (1.0f / 3.0f), c2 = (rr * rr) * (rr * rr) * (2.0f / 15.0f);
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const float u = st[t][e] * st[t][e];
                        st[t][e] *= fmaf(fmaf(u, c2, c1), u, 1.0f);
                    }
            } else if (MODS && alibi_on) {
                const float back = cap / a.scale;
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        st[t][e] = scaled_tanh_fast(st[t][e], k2, back, -2.0f * back);
            } else {
                lg_mul = 2.0f * cap * kLog2e;
                lg_add = cap * kLog2e;
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        st[t][e] = __builtin_amdgcn_rcpf(-1.0f - __builtin_amdgcn_exp2f(st[t][e] * k2));
            }
        }
        // Mask only blocks some row does not see whole: past the first row's
        // position (causal), or not inside every row's window or sink range.
        float cst = 0.0f;
        if constexpr (MODS) {
            // ALiBi (after the softcap): this lane's part of the bias, in
            // raw-product units, and the per-key part, one FMA per score.
            float sslope = 0.0f;
            if (alibi_on) {
                const bool right = k0 >= pos;
                sslope = right ? -slope_raw : slope_raw;
                cst = sslope * (float)(k0 + 4 * half - pos);
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        st[t][e] = fmaf(sslope, (float)(32 * t + 8 * (e >> 2) + (e & 3)), st[t][e]);
            }
            // A block crossing a non-causal row's position took the left-hand
            // form: keys right of the position are corrected to the mirror
            // image (causal rows never see them).
            if (alibi_on && !causal && k0 < pos && k0 + kBN - 1 > pos) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int j = k0 + 32 * t + 8 * (e >> 2) + 4 * half + (e & 3);
                        if (j > pos)
                            st[t][e] -= 2.0f * slope_raw * (float)(j - pos);
                    }
            }
            // Mask bits on every score of a partial block; otherwise only
            // blocks some row does not see whole (non-causal rows: keys past
            // the context).
            if ((mrow && part) || k0 + kBN - 1 > (causal ? pos_lo : key_hi) ||
                !(W <= 0 || k0 > pos_hi - W || k0 + kBN - 1 < S)) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int jo = 32 * t + 8 * (e >> 2) + 4 * half + (e & 3);
                        const int j = k0 + jo;
                        const uint32_t mw = t ? mw1 : mw0;
                        const bool vis = j <= posv && (W <= 0 || j > pos - W || j < S) && ((mw >> (jo & 31)) & 1u);
                        if (!vis)
                            st[t][e] = -INFINITY;
                    }
            }
        } else {
        const bool all_causal = k0 + kBN - 1 <= pos_lo;
        const bool all_window = W <= 0 || k0 > pos_hi - W || k0 + kBN - 1 < S;
        if (!(all_causal && all_window)) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int j = k0 + 32 * t + 8 * (e >> 2) + 4 * half + (e & 3);
                    const bool vis = j <= pos && (W <= 0 || j > pos - W || j < S);
                    if (!vis)
                        st[t][e] = -INFINITY;
                }
        }
        }

        // Online softmax (lane = one row, two lane halves share it).
        float mx = st[0][0];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                mx = fmaxf(mx, st[t][e]);
        if constexpr (MODS)
            mx += cst;
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_blk = fmaf(mx, lg_mul, lg_add);
        if (m_blk > m_ref + kRescaleSlack) {
            const float alpha = fast_exp2(m_ref - m_blk);
            l_part *= alpha;
#pragma unroll
            for (int t = 0; t < DT; ++t)
                acc[t] *= alpha;
            m_ref = m_blk;
        }
        const float msafe = m_ref == -INFINITY ? 0.0f : m_ref;
        const float p_off = MODS ? fmaf(cst, lg_mul, lg_add - msafe) : lg_add - msafe;

        // P^T as the B operand: tile t, k-step ks -> elements 8ks..8ks+7,
        // packed two fp16 values per 32-bit word.  The row sum is taken over
        // the same fp16 values the P.V product uses (one dot2 per pair).
        u32x4 pw[2][2];
        const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                const float p0 = fast_exp2(fmaf(st[t][e], lg_mul, p_off));
                const float p1 = fast_exp2(fmaf(st[t][e + 1], lg_mul, p_off));
                const f16x2 ph = __builtin_convertvector(f32x2{p0, p1}, f16x2);
                l_part = __builtin_amdgcn_fdot2(ph, ones, l_part, false);
                pw[t][e >> 3][(e & 7) >> 1] = __builtin_bit_cast(uint32_t, ph);
            }
        }

        // O^T += V^T P^T.  A operand via transposed LDS reads: lane 16q+j loads
        // V[key0 + j/4][d0 + 4(j%4) .. +3] and receives V[key0 + k][d0 + j] (k=0..3).
        const int q16 = lane >> 4;
        const int j16 = lane & 15;
        __builtin_amdgcn_s_setprio(1);
        // Output tiles innermost: consecutive products go to different
        // accumulators.
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const int key0 = 32 * t + 16 * ks + 4 * half + (j16 >> 2);
                    const int dim0 = 32 * dt + 16 * (q16 & 1) + 4 * (j16 & 3);
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)(&sm.v[cur][key0][dim0]));
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)(&sm.v[cur][key0 + 8][dim0]));
                    // Whole-vector concatenation: extracting the read's 16-bit
                    // elements one by one is mis-compiled by this toolchain
                    // (the operand gets splatted halves).
                    const f16x8 va = __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    const f16x8 pb = __builtin_bit_cast(f16x8, pw[t][ks]);
                    acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb, acc[dt], 0, 0, 0);
                }
            }
        }
        // Transposed V reads run six ahead, then two per product.
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int i = 0; i < (8 * DT - 6) / 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * DT - (8 * DT - 6) / 2, 0);

        __builtin_amdgcn_s_setprio(0);

        if (more)
            stash(cur ^ 1);
        __syncthreads();
        if constexpr (MODS) {
            mw0 = nw0;
            mw1 = nw1;
        }
    }

    // Epilogue: O = O^T / l, lse = (m + log2 l) ln 2.
    const float l_row = l_part + __shfl_xor(l_part, 32);
    if (a.split_blocks > 0) {
        if (!row_ok)
            return;
        // Partial state of this split (log2-unit reference max, sum,
        // unnormalised accumulator), merged by the LSE merge pass.
        const int64_t slot = (((int64_t)b * a.q_len + qi) * a.hq + h) * a.max_splits + split;
        float *pacc = a.ws_acc + slot * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
                *reinterpret_cast<f32x4 *>(pacc + 32 * dt + 8 * e4 + 4 * half) =
                    f32x4{acc[dt][4 * e4 + 0], acc[dt][4 * e4 + 1], acc[dt][4 * e4 + 2], acc[dt][4 * e4 + 3]};
        if (half == 0) {
            a.ws_ml[slot * 2 + 0] = m_ref;
            a.ws_ml[slot * 2 + 1] = l_row;
        }
        return;
    }
    // The output goes through LDS (the tile buffers are free after the loop's
    // last barrier): each wave stages its 32 rows one 32-dim tile at a time
    // and writes whole 128-byte row pieces (full cache lines) instead of
    // 32-byte pieces of 32 rows.  Non-temporal: the output goes to HBM while
    // this compute-bound kernel runs instead of lingering dirty in the cache.
    const bool any = l_row > 0.0f;
    const float inv = any ? 1.0f / l_row : __builtin_nanf("");
    constexpr int kSt = 36;  // staged row stride (floats): 144 bytes, conflict-free 16-byte writes
    static_assert(sizeof(sm) >= sizeof(float) * kWaves * 32 * kSt, "output staging fits the tile buffers");
    float *stage = reinterpret_cast<float *>(&sm) + wave * (32 * kSt);
    const int sr = lane >> 3;        // first staged row this lane stores (then + 8, + 16, + 24)
    const int sc = (lane & 7) * 4;   // its 4 dims of the tile
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
            *reinterpret_cast<f32x4 *>(stage + (lane & 31) * kSt + 8 * e4 + 4 * half) =
                f32x4{acc[dt][4 * e4 + 0] * inv, acc[dt][4 * e4 + 1] * inv, acc[dt][4 * e4 + 2] * inv,
                       acc[dt][4 * e4 + 3] * inv};
        __syncthreads();
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
            const int rr = sr + 8 * k4;
            const int r2 = wave * 32 + rr;
            const int ri2 = r2 / G;
            const int rj2 = r2 - ri2 * G;
            const int qi2 = i0 + ri2;
            if (ri2 < npos && qi2 < i1 && rj2 < gsize) {
                const int h2 = a.groups.list[gstart + rj2];
                const f32x4 o = *reinterpret_cast<const f32x4 *>(stage + rr * kSt + sc);
                __builtin_nontemporal_store(
                    o, reinterpret_cast<f32x4 *>(a.out + (((int64_t)b * a.q_len + qi2) * a.hq + h2) * D + 32 * dt + sc));
            }
        }
        __syncthreads();
    }
    if (a.lse && row_ok && half == 0)
        __builtin_nontemporal_store(any ? (m_ref + log2f(l_row)) * kLn2 : -INFINITY,
                                    a.lse + ((int64_t)b * a.q_len + qi) * a.hq + h);
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t stream)
{
    if (a.head_dim != 64 && a.head_dim != 128)
        return hipErrorNotSupported;
    if (a.groups.max_group < 1 || a.groups.max_group > kRows)
        return hipErrorNotSupported;
    const int npos = kRows / a.groups.max_group;
    PrefillArgs k = a;
    k.n_qblocks = (a.q_len + npos - 1) / npos;
    const int64_t blocks = (int64_t)k.n_qblocks * (a.split_blocks > 0 ? a.max_splits : 1) * a.batch * a.hkv;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    void (*kernel)(PrefillArgs);
    if (a.head_dim == 64)
        kernel = a.mods.any ? prefill_kernel<64, true, false>
                 : (a.softcap ? prefill_kernel<64, false, true> : prefill_kernel<64, false, false>);
    else
        kernel = a.mods.any ? prefill_kernel<128, true, false>
                 : (a.softcap ? prefill_kernel<128, false, true> : prefill_kernel<128, false, false>);
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(512), 0, stream, k);
    return hipGetLastError();
}

}  // namespace atlas

// prefill_split.hip -- tiled causal prefill for fp32 Q/K/V on the gfx950
// fp16 matrix cores, with every operand split into two fp16 parts.
//
// CPUAttn README: the method is defined on FP32 tensors, and its parallel
// lowering is the fused QK -> RowNorm -> PV tile pipeline whose causal mask
// stops each query block at its last reachable key block.  The fp32 matrix
// instructions of gfx950 run at one sixteenth of the fp16 rate, so this
// kernel keeps fp32 accuracy on the fp16 ones instead:
//
//   split      = an fp32 value x is carried as hi = fp16(x) and
//                lo = fp16(x - hi) (the subtraction is exact in fp32), so
//                hi + lo equals x to about 2^-22 relative, or to 2^-25
//                absolute where lo falls into the fp16 subnormal range;
//   range      = so that this absolute floor is negligible against the
//                row's own scale, every Q row and every K row is first
//                multiplied by the power of two that brings its largest
//                magnitude into [2^14, 2^15) (exact); the Q factor folds into
//                the row's exponent constant, the K factors (kept in LDS) are
//                applied to the 32 scores of each lane after the QK product.
//                V and P need no scaling: their floor is absolute and far
//                below the bar after the softmax weighting;
//   products   = x y is taken as hi_x hi_y + lo_x hi_y + hi_x lo_y on
//                v_mfma_f32_32x32x16_f16 (fp16 products are exact in the
//                fp32 accumulator; the dropped lo_x lo_y is below 2^-22 |x y|):
//                S^T = K Q^T with Q split once into registers and K split
//                while it is staged into LDS; P = 2^(s log2(e) scale - m) is
//                computed in fp32, summed in fp32 for the denominator and
//                split for O^T += V^T P^T, with V split while it is staged;
//   tiles      = as in the bf16 kernel: 256 rows (query position x q-head of
//                one K/V head) per 512-thread workgroup, 32 rows per wave,
//                64-key blocks, causal block-stop, window blocks skipped,
//                lazy rescaling (the reference max may lag by up to 2^8),
//                one LDS double buffer and one barrier per block, page ids
//                staged in LDS, heavy-first XCD-grouped grid;
//   softcap    = library tanhf (the hardware-exponential tanh of the bf16
//                kernel is too coarse for the fp32 bar).
//
// Modifications (MODS instances, atlas_attend_mods) as in the bf16 kernel:
// non-causal rows take every key block of the context; ALiBi bias (in the
// units the scores have after the softcap step) and mask bits per element.
//
// Precondition: |v| <= 65504 (fp16 range of V's hi parts; validation mode
// checks it).  Q and K rows take any magnitude below 2^115: the range shift
// (clamped to +-100) brings each row's largest element into [2^14, 2^15).
#include "device.h"
#include "kernels.h"

namespace atlas {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWaves = 8;
constexpr int kRows = 32 * kWaves;     // rows per workgroup
constexpr int kBN = 64;                // keys per block
constexpr int kPad = 24;               // row padding (elements): a 16-byte-odd row stride
constexpr float kRescaleSlack = 8.0f;  // log2 units the running max may lag
constexpr int kPidWindow = 1024;       // page ids staged in LDS at a time
constexpr int kMaxListed = 1024;       // candidate key blocks a mask can thin out (longer: all computed)

template <int D>
struct alignas(16) SplitSmem {
    alignas(16) uint16_t kh[2][kBN][D + kPad];  // fp16 bits of the K hi parts
    alignas(16) uint16_t kl[2][kBN][D + kPad];  // K lo parts
    alignas(16) uint16_t vh[2][kBN][D + kPad];  // V hi parts
    alignas(16) uint16_t vl[2][kBN][D + kPad];  // V lo parts
    alignas(16) float kscale[2][kBN];           // 2^-shift of each staged K row
    alignas(16) int32_t pid[kPidWindow];        // physical ids of pages [pid_base, pid_base + kPidWindow)
};

// Power-of-two shift that brings a largest magnitude m into [2^14, 2^15)
// (0 for m = 0; clamped so that 2^+-shift stays a normal fp32 number).
__device__ __forceinline__ int range_shift(float m)
{
    int e;
    frexpf(m, &e);  // m = f 2^e, f in [0.5, 1)
    const int s = 15 - e;
    return m > 0.0f ? (s < -100 ? -100 : (s > 100 ? 100 : s)) : 0;
}

__device__ __forceinline__ uint32_t f16bits2(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }

struct HiLo {
    uint32_t hi, lo;
};

// Two fp32 values -> (hi pair, lo pair) of fp16 bits.
__device__ __forceinline__ HiLo split2(float x0, float x1)
{
    const f16x2 h = __builtin_convertvector(f32x2{x0, x1}, f16x2);
    const f32x2 hf = __builtin_convertvector(h, f32x2);
    return {f16bits2(h), f16bits2(__builtin_convertvector(f32x2{x0 - hf[0], x1 - hf[1]}, f16x2))};
}

template <int D, bool MODS>
__global__ __launch_bounds__(512) void prefill_split_kernel(PrefillArgs a)
{
    constexpr int KS = D / 16;            // k-steps of the QK product
    constexpr int DT = D / 32;            // 32-dim tiles of the output
    constexpr int CPR = D / 4;            // 16-byte chunks (4 floats) per K/V row
    constexpr int CH = kBN * CPR / 512;   // chunks per thread per tile: 4 (D=128) or 2 (D=64)
    __shared__ SplitSmem<D> sm;

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
    const int W = a.window ? a.window[b] : 0;
    const int S = (a.sinks && W > 0) ? a.sinks[b] : 0;
    const float cap = a.softcap ? a.softcap[b] : 0.0f;
    // Last key any row of the block can see (the whole context when rows are
    // not causal).
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
    const int posv = causal ? pos : (row_ok ? ctx - 1 : -1);
    const uint32_t *mrow =
        (MODS && row_ok && a.mods.mask) ? a.mods.mask + ((int64_t)b * a.q_len + qi) * a.mods.mask_words : nullptr;

    // Q^T as the B operand, range-scaled and split: dims 16s + 8 half .. +7
    // of this lane's row (the other lane half holds the rest of the row).
    f16x8 qh[KS], ql[KS];
    float row_factor;  // 2^-shift of this row's Q scaling
    {
        const float *qrow = reinterpret_cast<const float *>(a.q) +
                            (((int64_t)b * a.q_len + (row_ok ? qi : 0)) * a.hq + h) * D;
        f32x4 x[2 * KS];
        float mx = 0.0f;
#pragma unroll
        for (int s = 0; s < 2 * KS; ++s) {
            x[s] = row_ok ? *reinterpret_cast<const f32x4 *>(qrow + 16 * (s >> 1) + 8 * half + 4 * (s & 1))
                          : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            mx = fmaxf(mx, fmaxf(fmaxf(fabsf(x[s][0]), fabsf(x[s][1])), fmaxf(fabsf(x[s][2]), fabsf(x[s][3]))));
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const int sh = range_shift(mx);
        row_factor = ldexpf(1.0f, -sh);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const f32x4 x0 = x[2 * s], x1 = x[2 * s + 1];
            const HiLo a0 = split2(ldexpf(x0[0], sh), ldexpf(x0[1], sh));
            const HiLo a1 = split2(ldexpf(x0[2], sh), ldexpf(x0[3], sh));
            const HiLo a2 = split2(ldexpf(x1[0], sh), ldexpf(x1[1], sh));
            const HiLo a3 = split2(ldexpf(x1[2], sh), ldexpf(x1[3], sh));
            qh[s] = __builtin_bit_cast(f16x8, u32x4{a0.hi, a1.hi, a2.hi, a3.hi});
            ql[s] = __builtin_bit_cast(f16x8, u32x4{a0.lo, a1.lo, a2.lo, a3.lo});
        }
    }

    const int ps = a.page_shift;
    const int pmask = (1 << ps) - 1;
    const float *kpages = reinterpret_cast<const float *>(a.k_pages);
    const float *vpages = reinterpret_cast<const float *>(a.v_pages);
    const int32_t *ptab = a.page_table + (int64_t)b * a.max_pages;

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

    // Global -> registers for key block kb (zeros past the last visible key):
    // thread t stages CH adjacent 16-byte pieces of one K row (then, in a
    // second phase, of the same V row).  K is fetched at the top of an
    // iteration and stashed after the QK products; V is fetched then and
    // stashed at the end, so only one tensor's staging registers are live.
    const int srow = (tid * CH) / CPR;
    const int scol = (tid * CH) - srow * CPR;
    f32x4 reg[CH];
    auto fetch = [&](const float *pages, int kb) {
        const int j = kb * kBN + srow;
        if (j <= key_hi) {
            const int pid = sm.pid[(j >> ps) - pid_base];
            const int64_t off = ((((int64_t)pid * a.hkv + g) << ps) + (j & pmask)) * D + scol * 4;
#pragma unroll
            for (int u = 0; u < CH; ++u)
                reg[u] = *reinterpret_cast<const f32x4 *>(pages + off + 4 * u);
        } else {
#pragma unroll
            for (int u = 0; u < CH; ++u)
                reg[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };
    // Registers -> the hi and lo rows of an LDS buffer.  K rows are first
    // range-scaled: the eight threads of a row (aligned lanes) share its
    // maximum, and its factor goes to kscale.
    auto stash = [&](uint16_t (*hi)[D + kPad], uint16_t (*lo)[D + kPad], float *kscale) {
        int sh = 0;
        if (kscale) {
            float mx = 0.0f;
#pragma unroll
            for (int u = 0; u < CH; ++u)
                mx = fmaxf(mx, fmaxf(fmaxf(fabsf(reg[u][0]), fabsf(reg[u][1])),
                                     fmaxf(fabsf(reg[u][2]), fabsf(reg[u][3]))));
            sh = range_shift(group_max<8>(mx));
            if ((tid & 7) == 0)
                kscale[srow] = ldexpf(1.0f, -sh);
        }
        uint32_t hw[2 * CH], lw[2 * CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            const HiLo x0 = split2(ldexpf(reg[u][0], sh), ldexpf(reg[u][1], sh));
            const HiLo x1 = split2(ldexpf(reg[u][2], sh), ldexpf(reg[u][3], sh));
            hw[2 * u] = x0.hi;
            lw[2 * u] = x0.lo;
            hw[2 * u + 1] = x1.hi;
            lw[2 * u + 1] = x1.lo;
        }
#pragma unroll
        for (int w4 = 0; w4 < CH / 2; ++w4) {
            const int col = scol * 4 + 8 * w4;
            *reinterpret_cast<u32x4 *>(&hi[srow][col]) = u32x4{hw[4 * w4], hw[4 * w4 + 1], hw[4 * w4 + 2], hw[4 * w4 + 3]};
            *reinterpret_cast<u32x4 *>(&lo[srow][col]) = u32x4{lw[4 * w4], lw[4 * w4 + 1], lw[4 * w4 + 2], lw[4 * w4 + 3]};
        }
    };

    // Scores leave the QK product in the row's scaled units (raw x 2^shift);
    // the softcap brings them back to raw units.
    const float c_log2 = cap > 0.0f ? a.scale * kLog2e : a.scale * kLog2e * row_factor;
    // MODS: ALiBi slope in the units of the scores after the softcap step.
    const float slope_u = (MODS && row_ok && a.mods.alibi)
                              ? a.mods.alibi[h] / (cap > 0.0f ? a.scale : a.scale * row_factor)
                              : 0.0f;
    float m_ref = -INFINITY;  // reference max (log2 units) the accumulator is scaled to
    float l_part = 0.0f;      // this lane-half's share of the softmax denominator (fp32)
    f32x16 acc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t)
        acc[t] = f32x16{};

#pragma unroll
    for (int s = 0; s < KS; ++s) {
        asm volatile("" : "+v"(qh[s]));
        asm volatile("" : "+v"(ql[s]));
    }

    // Key blocks the rows can see (sink blocks, then the window up to the
    // diagonal; every block up to the diagonal without a window).
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
    // (wave 0 compacts the flags with a ballot) by their index in the
    // candidate run, each marked full when every row's 64 bits are set (its
    // mask bits are then not applied per score).  The tests are
    // conservative: a listed block may still be wholly hidden by the causal
    // or window rule.  The flags live in the V tile buffer until the first
    // block is staged; the list (16-bit entries: index * 2 + partial) in
    // LDS of its own.
    __shared__ uint16_t s_lst[MODS ? kMaxListed : 1];
    __shared__ int32_t s_count;
    __shared__ int32_t s_pivot;
    const bool alibi_on = MODS && a.mods.alibi != nullptr;
    int n_run = n_iter;
    bool listed = false;
    // ALiBi: listed blocks whose first key is at or left of the last row's
    // position (the blocks run outward from the diagonal, see below).
    const int kb_diag = pos_hi >= 0 ? pos_hi / kBN : -1;
    int n_left = 0;
    if constexpr (MODS) {
        if (a.mods.mask && n_iter > 0 && n_iter <= kMaxListed) {
            listed = true;
            uint8_t *s_need = reinterpret_cast<uint8_t *>(&sm.vl[0][0][0]);
            uint8_t *s_part = s_need + kMaxListed;
            static_assert(sizeof(sm.vl) >= 2 * kMaxListed, "block flags fit the V lo buffer");
            for (int i = tid; i < n_iter; i += 512) {
                s_need[i] = 0;
                s_part[i] = 0;
            }
            __syncthreads();
            const int rows_pos = i1 - i0;
            const int wl = a.mods.mask_words - 1;
            const int total = n_iter * rows_pos;
            // kLoads (row, block) pairs per thread in flight at a time.
            constexpr int kLoads = 4;
            for (int base = 0; base < total; base += 512 * kLoads) {
                uint32_t m0[kLoads], m1[kLoads];
                int cc[kLoads], ww[kLoads];
#pragma unroll
                for (int u = 0; u < kLoads; ++u) {
                    const int idx = base + 512 * u + tid;
                    const int ix = idx < total ? idx : 0;
                    const int pp = ix / n_iter;
                    cc[u] = idx < total ? ix - pp * n_iter : -1;
                    const uint32_t *m = a.mods.mask + ((int64_t)b * a.q_len + i0 + pp) * a.mods.mask_words;
                    ww[u] = (block_at(ix - pp * n_iter) * kBN) >> 5;
                    m0[u] = m[ww[u] < wl ? ww[u] : wl];
                    m1[u] = m[ww[u] + 1 < wl ? ww[u] + 1 : wl];
                }
#pragma unroll
                for (int u = 0; u < kLoads; ++u) {
                    if (cc[u] < 0)
                        continue;
                    if ((m0[u] | m1[u]) != 0u)
                        s_need[cc[u]] = 1;
                    if ((m0[u] & m1[u]) != ~0u || ww[u] + 1 > wl)
                        s_part[cc[u]] = 1;
                }
            }
            __syncthreads();
            if (wave == 0) {
                int base = 0, left = 0;
                for (int c0 = 0; c0 < n_iter; c0 += 64) {
                    const int c = c0 + lane;
                    const bool f = c < n_iter && s_need[c];
                    const uint64_t bal = __ballot(f);
                    if (f)
                        s_lst[base + __popcll(bal & ((1ull << lane) - 1ull))] = (uint16_t)(c * 2 + s_part[c]);
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
        return block_at((MODS && listed) ? s_lst[i] >> 1 : i);
    };
    auto is_partial = [&](int it) { return !(MODS && listed) || (s_lst[list_at(it)] & 1); };
    // First page to stage for block kb when the walk goes backwards from it.
    auto back_first = [&](int kbx) { return ((kbx * kBN + kBN - 1) >> ps) - kPidWindow + 1; };

    if (n_run > 0)
        stage_pids(d_last >= 0 ? back_first(run_block(0)) : (run_block(0) * kBN) >> ps);
    __syncthreads();  // page ids staged; block flags no longer read
    if (n_run > 0) {
        fetch(kpages, run_block(0));
        stash(sm.kh[0], sm.kl[0], sm.kscale[0]);
        fetch(vpages, run_block(0));
        stash(sm.vh[0], sm.vl[0], nullptr);
    }
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
        if (more)
            fetch(kpages, kb_next);
        // MODS: the row's mask words for the block's two 32-key tiles (words
        // past the row's end hold keys beyond every context and are
        // clamped); full blocks need none.
        const bool part = is_partial(it);
        uint32_t mw0 = ~0u, mw1 = ~0u;
        if (MODS && mrow && part) {
            const int w = (kb * kBN) >> 5;
            const int wl = a.mods.mask_words - 1;
            mw0 = mrow[w < wl ? w : wl];
            mw1 = mrow[w + 1 < wl ? w + 1 : wl];
        }

        // S^T for the block: two 32-key tiles, three split products per
        // k-step; consecutive products alternate between the two tiles.
        __builtin_amdgcn_s_setprio(1);
        f32x16 st[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            f16x8 kfh[2], kfl[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                kfh[t] = *reinterpret_cast<const f16x8 *>(&sm.kh[cur][32 * t + (lane & 31)][16 * s + 8 * half]);
                kfl[t] = *reinterpret_cast<const f16x8 *>(&sm.kl[cur][32 * t + (lane & 31)][16 * s + 8 * half]);
            }
#pragma unroll
            for (int t = 0; t < 2; ++t)
                st[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kfh[t], qh[s], st[t], 0, 0, 0);
#pragma unroll
            for (int t = 0; t < 2; ++t)
                st[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kfl[t], qh[s], st[t], 0, 0, 0);
#pragma unroll
            for (int t = 0; t < 2; ++t)
                st[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kfh[t], ql[s], st[t], 0, 0, 0);
        }
        // K operand reads one k-step (four reads) ahead of their products.
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < KS - 1; ++i) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);

        __builtin_amdgcn_s_setprio(0);

        // The other buffer was last read before the previous barrier.
        if (more) {
            stash(sm.kh[cur ^ 1], sm.kl[cur ^ 1], sm.kscale[cur ^ 1]);
            fetch(vpages, kb_next);
        }

        // Undo the K rows' range scaling: lane half h holds keys
        // 32t + 8g + 4h + {0..3} in elements 4g .. 4g + 3 of tile t.
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 f = *reinterpret_cast<const f32x4 *>(&sm.kscale[cur][32 * t + 8 * g4 + 4 * half]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    st[t][4 * g4 + i] *= f[i];
            }

        // Softcap (before the mask), from the row's scaled units to the units
        // of the raw product.
        if (cap > 0.0f) {
            const float inv = row_factor * a.scale / cap, back = cap / a.scale;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    st[t][e] = back * tanhf(st[t][e] * inv);
        }
        const int k0 = kb * kBN;
        if constexpr (MODS) {
            // ALiBi: linear in j on blocks wholly on one side of this row's
            // position (one FMA with a constant per element), the absolute
            // value only on blocks crossing it.
            if (slope_u != 0.0f) {
                if (k0 + kBN - 1 <= pos) {
                    const float c = slope_u * (float)(k0 + 4 * half - pos);
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            st[t][e] += fmaf(slope_u, (float)(32 * t + 8 * (e >> 2) + (e & 3)), c);
                } else if (k0 >= pos) {
                    const float c = slope_u * (float)(pos - k0 - 4 * half);
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            st[t][e] += fmaf(-slope_u, (float)(32 * t + 8 * (e >> 2) + (e & 3)), c);
                } else {
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int j = k0 + 32 * t + 8 * (e >> 2) + 4 * half + (e & 3);
                            st[t][e] -= slope_u * fabsf((float)(pos - j));
                        }
                }
            }
        }
        // Mask only blocks some row does not see whole (and, with mask bits,
        // every block).
        const bool all_causal = k0 + kBN - 1 <= (causal ? pos_lo : key_hi);
        const bool all_window = W <= 0 || k0 > pos_hi - W || k0 + kBN - 1 < S;
        if (!(all_causal && all_window) || (MODS && mrow && part)) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int jo = 32 * t + 8 * (e >> 2) + 4 * half + (e & 3);
                    const int j = k0 + jo;
                    bool vis = j <= posv && (W <= 0 || j > pos - W || j < S);
                    if constexpr (MODS)
                        vis = vis && (((t ? mw1 : mw0) >> (jo & 31)) & 1u);
                    if (!vis)
                        st[t][e] = -INFINITY;
                }
        }

        // Online softmax (lane = one row, two lane halves share it).
        float mx = st[0][0];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                mx = fmaxf(mx, st[t][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_blk = mx * c_log2;
        if (m_blk > m_ref + kRescaleSlack) {
            const float alpha = fast_exp2(m_ref - m_blk);
            l_part *= alpha;
#pragma unroll
            for (int t = 0; t < DT; ++t)
                acc[t] *= alpha;
            m_ref = m_blk;
        }
        const float msafe = m_ref == -INFINITY ? 0.0f : m_ref;

        // P^T as split B operands: tile t, k-step ks -> elements 8ks..8ks+7.
        uint32_t ph[2][2][4], pl[2][2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int e = 0; e < 16; e += 2) {
                const float p0 = fast_exp2(fmaf(st[t][e], c_log2, -msafe));
                const float p1 = fast_exp2(fmaf(st[t][e + 1], c_log2, -msafe));
                l_part += p0 + p1;
                const HiLo pp = split2(p0, p1);
                ph[t][e >> 3][(e & 7) >> 1] = pp.hi;
                pl[t][e >> 3][(e & 7) >> 1] = pp.lo;
            }
        }

        // O^T += V^T P^T, split: per pair of output tiles, hi.hi, lo.hi and
        // hi.lo products alternating between the two accumulators.  V^T via
        // transposed LDS reads: lane 16q+j loads V[key0 + j/4][d0 + 4(j%4) .. +3]
        // and receives V[key0 + k][d0 + j] (k=0..3).
        const int q16 = lane >> 4;
        const int j16 = lane & 15;
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const f16x8 pbh = __builtin_bit_cast(f16x8, u32x4{ph[t][ks][0], ph[t][ks][1], ph[t][ks][2], ph[t][ks][3]});
                const f16x8 pbl = __builtin_bit_cast(f16x8, u32x4{pl[t][ks][0], pl[t][ks][1], pl[t][ks][2], pl[t][ks][3]});
                const int key0 = 32 * t + 16 * ks + 4 * half + (j16 >> 2);
#pragma unroll
                for (int dp = 0; dp < DT; dp += 2) {
                    f16x8 vah[2], val[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int dim0 = 32 * (dp + u) + 16 * (q16 & 1) + 4 * (j16 & 3);
                        const i16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(&sm.vh[cur][key0][dim0]));
                        const i16x4 h1 =
                            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(&sm.vh[cur][key0 + 8][dim0]));
                        const i16x4 l0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(&sm.vl[cur][key0][dim0]));
                        const i16x4 l1 =
                            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(&sm.vl[cur][key0 + 8][dim0]));
                        // Whole-vector concatenation (element-wise extraction
                        // of these reads is mis-compiled by this toolchain).
                        vah[u] = __builtin_bit_cast(f16x8, __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7));
                        val[u] = __builtin_bit_cast(f16x8, __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7));
                    }
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        acc[dp + u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vah[u], pbh, acc[dp + u], 0, 0, 0);
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        acc[dp + u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(val[u], pbh, acc[dp + u], 0, 0, 0);
#pragma unroll
                    for (int u = 0; u < 2; ++u)
                        acc[dp + u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vah[u], pbl, acc[dp + u], 0, 0, 0);
                }
            }
        }
        // Each group of six products (one pair of output tiles) has its eight
        // transposed reads issued during the previous group.
        constexpr int kGroups = 4 * (DT / 2);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int i = 0; i < kGroups - 1; ++i) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);

        __builtin_amdgcn_s_setprio(0);

        if (more)
            stash(sm.vh[cur ^ 1], sm.vl[cur ^ 1], nullptr);
        __syncthreads();
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

hipError_t launch_prefill_split(const PrefillArgs &a, hipStream_t stream)
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
        kernel = a.mods.any ? prefill_split_kernel<64, true> : prefill_split_kernel<64, false>;
    else
        kernel = a.mods.any ? prefill_split_kernel<128, true> : prefill_split_kernel<128, false>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(512), 0, stream, k);
    return hipGetLastError();
}

}  // namespace atlas

// atlas_api.cpp -- the C ABI declared in include/atlas.h.
//
// Validates every host-visible argument before anything is launched (on an
// error nothing is launched and no output is touched: the CFR-Atlas README,
// "Validation and hardening", asks for checked layout arithmetic and
// rejection of invalid configuration), builds the q-head <-> K/V-head groups,
// plans the split-KV grid and dispatches to the kernels.  A shape with no
// kernel returns ATLAS_ERR_UNSUPPORTED; there is no fallback path (ferrox-core
// "kernel_registry": a missing kernel is loud, not silently slow).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/atlas.h"
#include "kernels.h"
#include "plan.h"
#include "status.h"

namespace atlas {

namespace {
thread_local char g_last_error[512] = "";
}

int32_t fail(int32_t status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

int32_t ok()
{
    g_last_error[0] = '\0';
    return ATLAS_OK;
}

const char *last_error() { return g_last_error; }

}  // namespace atlas

namespace {

using atlas::fail;
using atlas::ok;

bool validate_mode()
{
    const char *v = std::getenv("ATLAS_VALIDATE");
    return v && v[0] && std::strcmp(v, "0") != 0;
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int64_t x)
{
    int s = 0;
    while ((int64_t(1) << s) < x)
        ++s;
    return s;
}

// Checked a*b for non-negative operands; false on int64 overflow.
bool mul_ok(int64_t a, int64_t b, int64_t *out)
{
    if (a < 0 || b < 0)
        return false;
    if (a != 0 && b > INT64_MAX / a)
        return false;
    *out = a * b;
    return true;
}

enum class Path { SplitValu, SplitMfma, TiledPrefill, TiledSplit };

// Everything derived from the arguments before launching.
struct Plan {
    atlas::HeadGroups groups;
    int page_shift = 0;
    int max_context = 0;
    int rows_per_item = 1;
    int n_chunks = 1;
    int split_tokens = 0;
    int max_splits = 0;
    int64_t rows_total = 0;
    int tiled_npos = 0;       // tiled paths: query positions per workgroup
    int split_blocks = 0;     // tiled paths: key blocks per split (0: no key splits)
    size_t workspace = 0;
    Path path = Path::SplitValu;
};

constexpr size_t kWorkspaceHeader = 256;  // validation-mode flags live here
constexpr int kDefaultSplitTokens = 4096; // keys per split-KV work item by default
constexpr int kMinItemsVector = 2048;     // work items (8 per CU) the vector fold's large plans aim at
constexpr int kMinItemsMatrix = 512;      // work items (2 per CU) the other plans aim at
constexpr int kSingleSplitKeys = 256;     // contexts up to this length take one split per row (no merge)
constexpr int kMinSplitTokens = 128;      // shortest default split
constexpr int kMaxSplitsPerRow = 32;      // default splits lengthen until a row has at most this many (more for calls with few items)
constexpr int kFillItems = 512;           // work items (two per CU) below which row chunks shrink

int32_t check_shapes(const atlas_attn_args *a, bool decode, Plan *p)
{
    if (!a)
        return fail(ATLAS_ERR_NULL, "args is NULL");
    const bool qf = a->q_dtype == ATLAS_DTYPE_F32, qb = a->q_dtype == ATLAS_DTYPE_BF16;
    const bool kvf = a->kv_dtype == ATLAS_DTYPE_F32, kvb = a->kv_dtype == ATLAS_DTYPE_BF16;
    if (!(qf && kvf) && !(qb && kvb) && !(qf && kvb))
        return fail(ATLAS_ERR_UNSUPPORTED,
                    "(q_dtype, kv_dtype) = (%d, %d) has no kernel: (f32, f32), (bf16, bf16) or (f32, bf16) "
                    "(f32=0, bf16=1)", a->q_dtype, a->kv_dtype);
    if (a->batch < 1 || a->q_len < 1 || a->num_q_heads < 1 || a->num_kv_heads < 1)
        return fail(ATLAS_ERR_SHAPE, "batch, q_len, num_q_heads, num_kv_heads must be >= 1");
    if (decode && a->q_len != 1)
        return fail(ATLAS_ERR_SHAPE, "atlas_attend_decode takes q_len == 1 (got %d)", a->q_len);
    if (a->num_q_heads > atlas::kMaxHeads || a->num_kv_heads > atlas::kMaxHeads)
        return fail(ATLAS_ERR_UNSUPPORTED, "at most %d q-heads and K/V heads", atlas::kMaxHeads);
    if (a->head_dim != 64 && a->head_dim != 128)
        return fail(ATLAS_ERR_UNSUPPORTED, "head_dim %d has no kernel (64 or 128)", a->head_dim);
    if (a->page_size < 1)
        return fail(ATLAS_ERR_SHAPE, "page_size must be >= 1");
    if (!is_pow2(a->page_size) || a->page_size > 4096)
        return fail(ATLAS_ERR_UNSUPPORTED, "page_size %d: powers of two up to 4096 only", a->page_size);
    if (a->num_phys_pages < 1 || a->max_pages_per_seq < 1)
        return fail(ATLAS_ERR_SHAPE, "num_phys_pages and max_pages_per_seq must be >= 1");
    if (!std::isfinite(a->scale) || !(a->scale > 0.0f))
        return fail(ATLAS_ERR_RANGE, "scale must be finite and > 0");

    int64_t max_ctx = 0;
    if (!mul_ok(a->max_pages_per_seq, a->page_size, &max_ctx) || max_ctx > INT32_MAX / 2)
        return fail(ATLAS_ERR_RANGE, "max_pages_per_seq * page_size overflows");
    if (a->q_len > max_ctx)
        return fail(ATLAS_ERR_RANGE, "q_len %d exceeds the largest context %lld", a->q_len,
                    (long long)max_ctx);
    int64_t arena_elems = 0, t = 0;
    if (!mul_ok(a->num_phys_pages, a->num_kv_heads, &t) || !mul_ok(t, a->page_size, &t) ||
        !mul_ok(t, a->head_dim, &arena_elems))
        return fail(ATLAS_ERR_RANGE, "arena size overflows");
    int64_t rows = 0;
    if (!mul_ok(a->batch, a->q_len, &t) || !mul_ok(t, a->num_q_heads, &rows) || rows > INT32_MAX)
        return fail(ATLAS_ERR_RANGE, "batch * q_len * num_q_heads must stay below 2^31");
    if ((int64_t)a->batch * a->max_pages_per_seq > INT32_MAX)
        return fail(ATLAS_ERR_RANGE, "page table larger than 2^31 entries");
    if (a->batch > 65535 || a->max_pages_per_seq > 65535 * 16)
        return fail(ATLAS_ERR_RANGE, "batch must be <= 65535 and max_pages_per_seq <= 1048560");

    // Head groups.
    const int hq = a->num_q_heads, hkv = a->num_kv_heads;
    int map[atlas::kMaxHeads];  // no host allocation on the call path
    if (a->head_map) {
        for (int h = 0; h < hq; ++h) {
            if (a->head_map[h] < 0 || a->head_map[h] >= hkv)
                return fail(ATLAS_ERR_SHAPE, "head_map[%d] = %d outside [0, %d)", h, a->head_map[h], hkv);
            map[h] = a->head_map[h];
        }
    } else {
        if (hq % hkv != 0)
            return fail(ATLAS_ERR_SHAPE, "num_q_heads %d not a multiple of num_kv_heads %d (pass head_map)",
                        hq, hkv);
        for (int h = 0; h < hq; ++h)
            map[h] = h / (hq / hkv);
    }
    std::memset(&p->groups, 0, sizeof p->groups);
    int pos = 0, gmax = 0;
    for (int g = 0; g < hkv; ++g) {
        p->groups.start[g] = (int16_t)pos;
        int n = 0;
        for (int h = 0; h < hq; ++h)
            if (map[h] == g) {
                p->groups.list[pos++] = (int16_t)h;
                p->groups.group_of[h] = (int16_t)g;
                p->groups.slot_of[h] = (int16_t)n++;
            }
        gmax = n > gmax ? n : gmax;
    }
    p->groups.start[hkv] = (int16_t)pos;
    p->groups.max_group = gmax;

    p->page_shift = log2i(a->page_size);
    p->max_context = (int)max_ctx;
    p->rows_total = rows;

    // Path: the tiled kernels for prefills with one dtype throughout
    // (window / sinks / softcap included; fp32 on split fp16 operands) from
    // 64 queries on, and below that when the split-KV kernels would need
    // several row chunks per K/V head (queries x largest group above 32 rows
    // for a bf16 cache, 16 rows per chunk; above 8 for fp32, at most 8 per
    // chunk) and the call is large enough (batch x queries x key bound at
    // least 2^17, or 2^16 for fp32 with two or more queries); else the
    // split-KV kernels (matrix cores for a bf16 cache, an fp32 query
    // included; vector ALUs for fp32).  Decode calls always take the
    // split-KV kernels, so that they match the fused-regeneration decode
    // (which only those kernels implement) bit for bit; one query through
    // the prefill entry follows the rule above.  Each row chunk of a split kernel re-reads its K/V head's
    // keys, so its time grows with the chunk count, while a tiled query block
    // covers up to 256 rows in one pass over the keys.  Measured with 3 to 48
    // queries, groups of 1, 4 and 8, over 2048 to 32768 keys (1 and 4
    // sequences): the tiled kernels were up to 2.8x (bf16) and 9.6x (fp32)
    // faster from 3 chunks (bf16) or 2 chunks (fp32) on (fp32, 4 x 48
    // queries over 32768 keys: 3877 -> 405 us), and up to 47 % (bf16) and
    // 96 % (fp32) slower with fewer chunks; below the size bounds the split
    // kernels were up to 26 % faster (one sequence of 16 fp32 queries over
    // 2048 keys).  One query (1 to 16 sequences over 8192 to 131072 keys, 48
    // to 128 q-heads over 1 or 2 K/V heads for bf16, 16 to 128 over 1 to 8
    // for fp32): the tiled kernels up to 2.0x (bf16, 8 x 128 q-heads over
    // one K/V head at 32768 keys, 86.9 -> 46.5 us) and 2.3x faster (fp32) at
    // 2^17 pairs and above (within 5 % either way on the largest fp32
    // calls, 8 to 16 sequences of 131072 keys over 4 or 8 K/V heads), and up
    // to 93 % slower (fp32) below: their fixed cost is spread over few rows.
    const int64_t pairs = (int64_t)a->batch * a->q_len * max_ctx;
    const int64_t head_rows = (int64_t)a->q_len * gmax;
    const int64_t min_pairs = (kvb || a->q_len == 1) ? (INT64_C(1) << 17) : (INT64_C(1) << 16);
    const bool tile = a->q_len >= 64 || (head_rows > (kvb ? 32 : 8) && pairs >= min_pairs);
    if (!decode && qb && kvb && tile)
        p->path = Path::TiledPrefill;
    else if (!decode && qf && kvf && tile)
        p->path = Path::TiledSplit;
    else if (kvb)
        p->path = Path::SplitMfma;
    else
        p->path = Path::SplitValu;

    if (p->path == Path::TiledPrefill || p->path == Path::TiledSplit) {
        // Key splits when the grid would not fill the chip once (fewer
        // workgroups than CUs, e.g. a short prefill chunk behind a long
        // history): aim at about one round (one 512-thread workgroup per
        // CU), at least 8 key blocks (512 keys) per split, partial states
        // within 1 GiB.  Measured: four rounds of shorter runs spent a third
        // of a 128-query chunk's time writing and merging partial states
        // (139 against 90 us); a full round runs unsplit, since splitting it
        // only adds that traffic.
        p->workspace = kWorkspaceHeader;
        p->tiled_npos = 256 / gmax;
        const int64_t n_qblocks = (a->q_len + p->tiled_npos - 1) / p->tiled_npos;
        const int64_t wgs = n_qblocks * a->batch * hkv;
        const int64_t max_blocks = (max_ctx + 63) / 64;
        p->split_blocks = 0;
        p->max_splits = 1;
        if (wgs < 256 && max_blocks > 16) {
            const int64_t want = (256 + wgs - 1) / wgs;
            int64_t sb = std::max<int64_t>(8, (max_blocks + want - 1) / want);
            const int64_t per_split = rows * (int64_t)(a->head_dim + 2) * 4;
            while ((max_blocks + sb - 1) / sb > 1 && per_split * ((max_blocks + sb - 1) / sb) > (INT64_C(1) << 30))
                sb *= 2;
            const int64_t ms = (max_blocks + sb - 1) / sb;
            if (ms > 1) {
                p->split_blocks = (int)sb;
                p->max_splits = (int)ms;
                p->workspace += (size_t)(per_split * ms);
            }
        }
        return ok();
    }

    // Split-KV plan: rows of a K/V head per work item, then keys per split.
    int rpi = 1;
    if (p->path == Path::SplitMfma) {
        rpi = 16;  // the matrix-core fold always takes 16 rows (MFMA width)
    } else {
        while (rpi < head_rows && rpi < 8)
            rpi <<= 1;
        // Few rows over short contexts: smaller row chunks spread the call
        // over more CUs (each work item's fold is a serial chain of memory
        // round trips and per-key vector work, so fewer rows per item finish
        // sooner).  Counted at the shortest spans (64 keys).
        const int64_t spans_min = (max_ctx + 63) / 64;
        while (rpi > 1 && (int64_t)a->batch * hkv * ((head_rows + rpi - 1) / rpi) * spans_min < kFillItems)
            rpi >>= 1;
    }
    p->rows_per_item = rpi;
    p->n_chunks = (int)((head_rows + rpi - 1) / rpi);
    const int64_t items_per_split = (int64_t)a->batch * hkv * p->n_chunks;
    const int64_t max_t_by_lds = (int64_t)(atlas::kMaxSplitPages - 2) << p->page_shift;
    int64_t T;
    if (a->split_tokens != 0) {
        if (a->split_tokens < 1)
            return fail(ATLAS_ERR_RANGE, "split_tokens must be >= 0");
        T = a->split_tokens;
        if (T > max_t_by_lds)
            return fail(ATLAS_ERR_RANGE, "split_tokens %d spans more than %d pages", a->split_tokens,
                        atlas::kMaxSplitPages - 2);
    } else if (max_ctx <= kSingleSplitKeys && !a->sink_tokens && kSingleSplitKeys <= max_t_by_lds) {
        // Short contexts: one split per row, finished by the fold itself, so
        // no merge is launched.  Measured (C-ABI call, four shapes at 256
        // keys): 11.7-13.8 us with 64-key splits and the merge against
        // 8.7-11.9 us; at 512 keys the longer serial fold no longer pays for
        // every shape, at 1024 it loses.
        T = kSingleSplitKeys;
    } else {
        // Long spans amortise a work item's set-up (page ids, query, final
        // combine); shorter ones only while the call would have fewer work
        // items than it needs, down to 128 keys and to at most 32 splits per
        // row (more for calls with few work items, below): past those, the
        // per-split set-up and the merge's traffic cost more than the extra
        // work items gain.  The matrix-core fold
        // (bf16 K/V) starts at 4096 keys and wants two items per CU.  The
        // vector fold (fp32 K/V) keeps the plan for eight items per CU from
        // 4096 keys when that plan's splits are 1024 keys or longer (large
        // calls: the long-context decode, long fp32 prefills); otherwise it
        // takes two items per CU from 512 keys.  The plan does not depend on
        // whether the fold generates cold pages, so generating and reading
        // the same pages give the same bits.
        // Measured (C-ABI calls over 60 shapes of 1 to 128 rows per K/V head
        // and 512 to 32768 keys, and 60 fp32 reading and generating calls)
        // against halving from 4096 down to 64 keys for eight items per CU:
        // up to 1.8x faster for mid-size calls (16 fp32 queries x 8 q-heads
        // over 8192 keys 50.3 -> 27.8 us; a bf16 batch of 16 x 64 q-heads
        // over 2048 keys 53.2 -> 32.6 us; an fp32 batch of 8 x 64 q-heads
        // over 2048 keys 50.4 -> 40.3 us, generating 93.0 -> 74.1 us),
        // within run-to-run spread or a few per cent elsewhere.  Generating
        // fp32 decodes lost up to 44 % with splits of 2048 keys where 512
        // served (2 x 32768 keys 77.6 -> 112 us), hence the 512-key start.
        // Calls with few (sequence, K/V head, row chunk) items (one or two
        // sequences over few K/V heads) may take more than 32 splits per
        // row, as many as two work items per CU need: their rows are few, so
        // the merge's extra states cost little (past 64 splits a row is
        // merged by eight waves).  Measured: one sequence of 8 fp32 q-heads
        // over one K/V head and 131072 keys 275 -> 67 us, a bf16 one of 64
        // q-heads 69 -> 40 us.
        const int64_t max_splits_row =
            std::max<int64_t>(kMaxSplitsPerRow, (kFillItems + items_per_split - 1) / items_per_split);
        auto pick = [&](int64_t start, int64_t min_items) {
            int64_t t = start;
            while (t > kMinSplitTokens && items_per_split * ((max_ctx + t - 1) / t) < min_items)
                t /= 2;
            while (t < kDefaultSplitTokens && (max_ctx + t - 1) / t > max_splits_row)
                t *= 2;
            return t;
        };
        if (a->kv_dtype == ATLAS_DTYPE_BF16) {
            T = pick(kDefaultSplitTokens, kMinItemsMatrix);
        } else {
            T = pick(kDefaultSplitTokens, kMinItemsVector);
            if (T < 1024)
                T = pick(512, kMinItemsMatrix);
        }
        if (T > max_t_by_lds)
            T = max_t_by_lds;
    }
    p->split_tokens = (int)T;
    p->max_splits = atlas::max_splits_bound((int)max_ctx, (int)T, a->sink_tokens != nullptr);
    if (p->max_splits > atlas::kMaxMergeSplits || items_per_split / a->batch > 65535)
        return fail(ATLAS_ERR_RANGE, "split grid too large (raise split_tokens)");
    int64_t slots = 0, ws = 0;
    if (!mul_ok(rows, p->max_splits, &slots) || !mul_ok(slots, (int64_t)(a->head_dim + 2) * 4, &ws))
        return fail(ATLAS_ERR_RANGE, "workspace size overflows");
    p->workspace = kWorkspaceHeader + (size_t)ws;
    return ok();
}

int32_t check_pointers(const atlas_attn_args *a, const Plan &p)
{
    if (!a->q || !a->k_pages || !a->v_pages || !a->page_table || !a->context_lens || !a->out)
        return fail(ATLAS_ERR_NULL, "q, k_pages, v_pages, page_table, context_lens and out are required");
    if (p.workspace > 0) {
        if (!a->workspace)
            return fail(ATLAS_ERR_NULL, "workspace is required (%zu bytes)", p.workspace);
        if (a->workspace_bytes < p.workspace)
            return fail(ATLAS_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", a->workspace_bytes,
                        p.workspace);
        if (reinterpret_cast<uintptr_t>(a->workspace) % 16 != 0)
            return fail(ATLAS_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    }
    return ok();
}

// Validation mode: copy the device-resident lengths and page table to the
// host, check them, and scan the visible inputs for NaN/Inf.
int32_t validate_device(const atlas_attn_args *a, const Plan &p, hipStream_t stream, bool regen)
{
    const int B = a->batch;
    std::vector<int32_t> ctx(B), pt((size_t)B * a->max_pages_per_seq), win(B, 0), snk(B, 0);
    hipError_t e = hipMemcpyAsync(ctx.data(), a->context_lens, sizeof(int32_t) * B, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(pt.data(), a->page_table, sizeof(int32_t) * pt.size(), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess && a->window)
        e = hipMemcpyAsync(win.data(), a->window, sizeof(int32_t) * B, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess && a->sink_tokens)
        e = hipMemcpyAsync(snk.data(), a->sink_tokens, sizeof(int32_t) * B, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess)
        e = hipStreamSynchronize(stream);
    if (e != hipSuccess)
        return fail(ATLAS_ERR_DEVICE, "validation copy failed: %s", hipGetErrorString(e));
    for (int b = 0; b < B; ++b) {
        if (ctx[b] < a->q_len || ctx[b] > p.max_context)
            return fail(ATLAS_ERR_RANGE, "context_lens[%d] = %d outside [q_len=%d, %d]", b, ctx[b], a->q_len,
                        p.max_context);
        if (win[b] < 0 || snk[b] < 0)
            return fail(ATLAS_ERR_RANGE, "window/sink_tokens[%d] negative", b);
        const int np = (ctx[b] + a->page_size - 1) / a->page_size;
        for (int lp = 0; lp < np; ++lp) {
            const int32_t id = pt[(size_t)b * a->max_pages_per_seq + lp];
            if (regen && id == ATLAS_PAGE_REGENERATE)
                continue;
            if (id < 0 || id >= a->num_phys_pages)
                return fail(ATLAS_ERR_POOL, "page_table[%d][%d] = %d outside the pool of %d pages", b, lp, id,
                            a->num_phys_pages);
        }
    }
    // NaN/Inf scan of what the call will read; the flag word sits in the
    // workspace header.
    atlas::ScanArgs s{};
    s.q = a->q;
    s.k_pages = a->k_pages;
    s.v_pages = a->v_pages;
    s.page_table = a->page_table;
    s.context_lens = a->context_lens;
    s.flag = static_cast<int *>(a->workspace);
    s.batch = a->batch;
    s.q_len = a->q_len;
    s.hq = a->num_q_heads;
    s.hkv = a->num_kv_heads;
    s.head_dim = a->head_dim;
    s.page_shift = p.page_shift;
    s.num_phys = a->num_phys_pages;
    s.max_pages = a->max_pages_per_seq;
    s.max_context = p.max_context;
    s.check_f16 = (p.path == Path::TiledPrefill || p.path == Path::TiledSplit) ? 1 : 0;
    int flag = 0;
    e = hipMemsetAsync(s.flag, 0, sizeof(int), stream);
    if (e == hipSuccess)
        e = atlas::launch_scan(s, a->q_dtype, a->kv_dtype, stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(&flag, s.flag, sizeof(int), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess)
        e = hipStreamSynchronize(stream);
    if (e != hipSuccess)
        return fail(ATLAS_ERR_DEVICE, "validation scan failed: %s", hipGetErrorString(e));
    if (flag & 1)
        return fail(ATLAS_ERR_NONFINITE, "NaN or Inf in q or in the K/V rows the contexts cover");
    if (flag & 2)
        return fail(ATLAS_ERR_RANGE, "a V value exceeds 65504, the fp16 range of the tiled prefill's P.V "
                                     "product");
    return ok();
}

// In-kernel regeneration request of atlas_attend_decode_regen.
struct RegenSpec {
    uint64_t seed;
    int32_t layer;
    const int32_t *seq_keys;  // device [B] or null
};

// Host checks of atlas_attn_mods (NULL: none) and their kernel form.
int32_t check_mods(const atlas_attn_args *a, const Plan &p, const atlas_attn_mods *m, atlas::Mods *out)
{
    *out = atlas::Mods{};
    out->causal = 1;
    if (!m)
        return ok();
    if (m->causal != 0 && m->causal != 1)
        return fail(ATLAS_ERR_RANGE, "mods->causal must be 0 or 1 (got %d)", m->causal);
    if (!m->causal && (a->window || a->sink_tokens))
        return fail(ATLAS_ERR_UNSUPPORTED, "window and sink_tokens apply to causal rows only");
    if (m->mask_bits) {
        const int64_t need = ((int64_t)p.max_context + 31) / 32;
        if (m->mask_words < need)
            return fail(ATLAS_ERR_SHAPE, "mask_words %d < %lld (max_pages_per_seq * page_size / 32, rounded up)",
                        m->mask_words, (long long)need);
        int64_t t = 0;
        if (!mul_ok((int64_t)a->batch * a->q_len, m->mask_words, &t) || t > INT64_C(1) << 40)
            return fail(ATLAS_ERR_RANGE, "mask size overflows");
    }
    out->alibi = m->alibi_slopes;
    out->mask = m->mask_bits;
    out->mask_words = m->mask_bits ? m->mask_words : 0;
    out->causal = m->causal;
    out->any = (!m->causal || m->alibi_slopes || m->mask_bits) ? 1 : 0;
    return ok();
}

int32_t attend(const atlas_attn_args *a, void *stream_ptr, bool decode, const RegenSpec *regen = nullptr,
               const atlas_attn_mods *mods_in = nullptr)
{
    Plan p;
    int32_t st = check_shapes(a, decode, &p);
    if (st != ATLAS_OK)
        return st;
    atlas::Mods mods;
    st = check_mods(a, p, mods_in, &mods);
    if (st != ATLAS_OK)
        return st;
    if (regen) {
        if (regen->layer < 0 || regen->layer >= (1 << 16))
            return fail(ATLAS_ERR_RANGE, "layer must be in [0, 65536)");
    }
    st = check_pointers(a, p);
    if (st != ATLAS_OK)
        return st;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
    if (validate_mode()) {
        st = validate_device(a, p, stream, regen != nullptr);
        if (st != ATLAS_OK)
            return st;
        if (regen && regen->seq_keys) {
            std::vector<int32_t> keys(a->batch);
            hipError_t e = hipMemcpyAsync(keys.data(), regen->seq_keys, sizeof(int32_t) * a->batch,
                                          hipMemcpyDeviceToHost, stream);
            if (e == hipSuccess)
                e = hipStreamSynchronize(stream);
            if (e != hipSuccess)
                return fail(ATLAS_ERR_DEVICE, "validation copy failed: %s", hipGetErrorString(e));
            for (int b = 0; b < a->batch; ++b)
                if (keys[b] < 0 || keys[b] >= (1 << 16))
                    return fail(ATLAS_ERR_RANGE, "seq_keys[%d] = %d outside [0, 65536)", b, keys[b]);
        }
    }

    if (p.path == Path::TiledPrefill || p.path == Path::TiledSplit) {
        atlas::PrefillArgs k{};
        k.q = a->q;
        k.k_pages = a->k_pages;
        k.v_pages = a->v_pages;
        k.page_table = a->page_table;
        k.context_lens = a->context_lens;
        k.window = a->window;
        k.sinks = a->sink_tokens;
        k.softcap = a->softcap;
        k.out = a->out;
        k.lse = a->lse;
        k.batch = a->batch;
        k.q_len = a->q_len;
        k.hq = a->num_q_heads;
        k.hkv = a->num_kv_heads;
        k.head_dim = a->head_dim;
        k.page_shift = p.page_shift;
        k.num_phys = a->num_phys_pages;
        k.max_pages = a->max_pages_per_seq;
        k.max_context = p.max_context;
        k.scale = a->scale;
        k.mods = mods;
        k.groups = p.groups;
        k.split_blocks = p.split_blocks;
        k.max_splits = p.max_splits;
        if (p.split_blocks > 0) {
            char *ws = static_cast<char *>(a->workspace) + kWorkspaceHeader;
            k.ws_acc = reinterpret_cast<float *>(ws);
            k.ws_ml = reinterpret_cast<float *>(ws + (size_t)p.rows_total * p.max_splits * a->head_dim * sizeof(float));
        }
        if (std::getenv("ATLAS_DEBUG"))
            std::fprintf(stderr, "atlas: tiled prefill (%s) positions/block=%d split_blocks=%d max_splits=%d "
                                 "workspace=%zu\n",
                         p.path == Path::TiledPrefill ? "bf16" : "fp32", p.tiled_npos, p.split_blocks,
                         p.max_splits, p.workspace);
        hipError_t e = p.path == Path::TiledPrefill ? atlas::launch_prefill_mfma(k, stream)
                                                     : atlas::launch_prefill_split(k, stream);
        if (e == hipSuccess && p.split_blocks > 0) {
            // LSE merge of the key splits.
            atlas::SplitArgs m{};
            m.context_lens = a->context_lens;
            m.window = a->window;
            m.sinks = a->sink_tokens;
            m.ws_acc = k.ws_acc;
            m.ws_ml = k.ws_ml;
            m.out = a->out;
            m.lse = a->lse;
            m.batch = a->batch;
            m.q_len = a->q_len;
            m.hq = a->num_q_heads;
            m.hkv = a->num_kv_heads;
            m.head_dim = a->head_dim;
            m.max_context = p.max_context;
            m.split_tokens = 1;
            m.max_splits = p.max_splits;
            m.rows_per_item = 1;
            m.n_chunks = 1;
            m.tiled_blocks = p.split_blocks;
            m.tiled_npos = p.tiled_npos;
            m.mods = mods;
            m.groups = p.groups;
            e = atlas::launch_merge(m, stream);
        }
        if (e == hipErrorNotSupported)
            return fail(ATLAS_ERR_UNSUPPORTED, "no tiled prefill kernel for this shape");
        if (e != hipSuccess)
            return fail(ATLAS_ERR_DEVICE, "prefill launch: %s", hipGetErrorString(e));
        return ok();
    }

    atlas::SplitArgs k{};
    k.q = a->q;
    k.k_pages = a->k_pages;
    k.v_pages = a->v_pages;
    k.page_table = a->page_table;
    k.context_lens = a->context_lens;
    k.window = a->window;
    k.sinks = a->sink_tokens;
    k.softcap = a->softcap;
    char *ws = static_cast<char *>(a->workspace) + kWorkspaceHeader;
    const size_t acc_bytes = (size_t)p.rows_total * p.max_splits * a->head_dim * sizeof(float);
    k.ws_acc = reinterpret_cast<float *>(ws);
    k.ws_ml = reinterpret_cast<float *>(ws + acc_bytes);
    k.out = a->out;
    k.lse = a->lse;
    k.batch = a->batch;
    k.q_len = a->q_len;
    k.hq = a->num_q_heads;
    k.hkv = a->num_kv_heads;
    k.head_dim = a->head_dim;
    k.page_shift = p.page_shift;
    k.num_phys = a->num_phys_pages;
    k.max_pages = a->max_pages_per_seq;
    k.max_context = p.max_context;
    k.split_tokens = p.split_tokens;
    k.max_splits = p.max_splits;
    k.rows_per_item = p.rows_per_item;
    k.n_chunks = p.n_chunks;
    k.scale = a->scale;
    k.mods = mods;
    k.groups = p.groups;
    k.q_f32 = a->q_dtype == ATLAS_DTYPE_F32 ? 1 : 0;
    if (regen) {
        k.regen_seed = regen->seed;
        k.regen_layer = regen->layer;
        k.seq_keys = regen->seq_keys;
        k.regen = 1;
    }

    if (std::getenv("ATLAS_DEBUG"))
        std::fprintf(stderr,
                     "atlas: split-KV %s (%s) rows/item=%d chunks=%d split_tokens=%d max_splits=%d "
                     "workspace=%zu\n",
                     decode ? "decode" : "prefill", p.path == Path::SplitMfma ? "mfma" : "valu",
                     p.rows_per_item, p.n_chunks, p.split_tokens,
                     p.max_splits, p.workspace);

    hipError_t e = p.path == Path::SplitMfma ? atlas::launch_split_mfma(k, stream)
                                             : atlas::launch_split_valu(k, stream);
    if (e != hipSuccess)
        return fail(ATLAS_ERR_DEVICE, "split launch: %s", hipGetErrorString(e));
    // One split per row: the fold wrote the final rows (merge_row.h,
    // write_single_split).
    if (p.max_splits == 1)
        return ok();
    e = atlas::launch_merge(k, stream);
    if (e != hipSuccess)
        return fail(ATLAS_ERR_DEVICE, "merge launch: %s", hipGetErrorString(e));
    return ok();
}

size_t workspace_bytes(const atlas_attn_args *a, bool decode)
{
    Plan p;
    if (check_shapes(a, decode, &p) != ATLAS_OK)
        return SIZE_MAX;
    return p.workspace;
}

}  // namespace

extern "C" {

int32_t atlas_abi_version(void) { return ATLAS_ABI_VERSION; }

const char *atlas_status_str(int32_t status)
{
    switch (status) {
    case ATLAS_OK: return "ok";
    case ATLAS_ERR_NULL: return "null pointer";
    case ATLAS_ERR_SHAPE: return "invalid shape";
    case ATLAS_ERR_RANGE: return "value out of range";
    case ATLAS_ERR_UNSUPPORTED: return "unsupported (no kernel for this configuration)";
    case ATLAS_ERR_WORKSPACE: return "workspace too small or misaligned";
    case ATLAS_ERR_POOL: return "page id outside the physical pool";
    case ATLAS_ERR_NONFINITE: return "non-finite input";
    case ATLAS_ERR_DEVICE: return "HIP runtime error";
    default: return "unknown status";
    }
}

const char *atlas_last_error(void) { return atlas::last_error(); }

size_t atlas_decode_workspace_bytes(const atlas_attn_args *args) { return workspace_bytes(args, true); }

size_t atlas_prefill_workspace_bytes(const atlas_attn_args *args) { return workspace_bytes(args, false); }

int32_t atlas_attend_decode(const atlas_attn_args *args, void *stream) { return attend(args, stream, true); }

int32_t atlas_attend_prefill(const atlas_attn_args *args, void *stream) { return attend(args, stream, false); }

int32_t atlas_attend_mods(const atlas_attn_args *args, const atlas_attn_mods *mods, void *stream)
{
    return attend(args, stream, false, nullptr, mods);
}

int32_t atlas_attend_decode_regen(const atlas_attn_args *args, uint64_t seed, int32_t layer,
                                  const int32_t *seq_keys, void *stream)
{
    const RegenSpec r{seed, layer, seq_keys};
    return attend(args, stream, true, &r);
}

int32_t atlas_regenerate_pages(const atlas_regen_args *a, void *stream)
{
    if (!a)
        return fail(ATLAS_ERR_NULL, "args is NULL");
    if (a->dtype != ATLAS_DTYPE_F32 && a->dtype != ATLAS_DTYPE_BF16)
        return fail(ATLAS_ERR_UNSUPPORTED, "dtype %d has no kernel", a->dtype);
    if (a->head_dim != 64 && a->head_dim != 128)
        return fail(ATLAS_ERR_UNSUPPORTED, "head_dim %d has no kernel (64 or 128)", a->head_dim);
    if (a->page_size < 1 || a->num_kv_heads < 1 || a->num_phys_pages < 1 || a->num_jobs < 0)
        return fail(ATLAS_ERR_SHAPE, "page_size, num_kv_heads, num_phys_pages >= 1 and num_jobs >= 0 required");
    if (!is_pow2(a->page_size) || a->page_size > 4096)
        return fail(ATLAS_ERR_UNSUPPORTED, "page_size %d: powers of two up to 4096 only", a->page_size);
    if (a->layer < 0 || a->layer >= (1 << 16))
        return fail(ATLAS_ERR_RANGE, "layer must be in [0, 65536)");
    if (a->num_kv_heads >= (1 << 30))
        return fail(ATLAS_ERR_RANGE, "num_kv_heads must be below 2^30");
    int64_t t = 0;
    if (!mul_ok(a->num_phys_pages, a->num_kv_heads, &t) || !mul_ok(t, a->page_size, &t) ||
        !mul_ok(t, a->head_dim, &t))
        return fail(ATLAS_ERR_RANGE, "arena size overflows");
    if (a->num_jobs == 0)
        return ok();
    if (!a->jobs || !a->k_pages || !a->v_pages)
        return fail(ATLAS_ERR_NULL, "jobs, k_pages and v_pages are required");
    atlas::RegenArgs k{};
    k.seed = a->seed;
    k.jobs = reinterpret_cast<const int32_t *>(a->jobs);
    k.k_pages = a->k_pages;
    k.v_pages = a->v_pages;
    k.layer = a->layer;
    k.hkv = a->num_kv_heads;
    k.head_dim = a->head_dim;
    k.page_shift = log2i(a->page_size);
    k.num_phys = a->num_phys_pages;
    k.n_jobs = a->num_jobs;
    hipError_t e = atlas::launch_regen(k, a->dtype, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(ATLAS_ERR_DEVICE, "regen launch: %s", hipGetErrorString(e));
    return ok();
}

int32_t atlas_append_kv(const atlas_append_args *a, void *stream_ptr)
{
    if (!a)
        return fail(ATLAS_ERR_NULL, "args is NULL");
    if (a->dtype != ATLAS_DTYPE_F32 && a->dtype != ATLAS_DTYPE_BF16)
        return fail(ATLAS_ERR_UNSUPPORTED, "dtype %d has no kernel", a->dtype);
    if (a->head_dim != 64 && a->head_dim != 128)
        return fail(ATLAS_ERR_UNSUPPORTED, "head_dim %d has no kernel (64 or 128)", a->head_dim);
    if (a->batch < 1 || a->n_new < 0 || a->num_kv_heads < 1 || a->page_size < 1 || a->num_phys_pages < 1 ||
        a->max_pages_per_seq < 1)
        return fail(ATLAS_ERR_SHAPE, "batch, num_kv_heads, page_size, num_phys_pages, max_pages_per_seq >= 1 "
                                     "and n_new >= 0 required");
    if (!is_pow2(a->page_size) || a->page_size > 4096)
        return fail(ATLAS_ERR_UNSUPPORTED, "page_size %d: powers of two up to 4096 only", a->page_size);
    int64_t t = 0;
    if (!mul_ok(a->num_phys_pages, a->num_kv_heads, &t) || !mul_ok(t, a->page_size, &t) ||
        !mul_ok(t, a->head_dim, &t) || !mul_ok(a->max_pages_per_seq, a->page_size, &t) || t > INT32_MAX ||
        !mul_ok(a->batch, a->n_new, &t) || !mul_ok(t, a->num_kv_heads, &t) || !mul_ok(t, a->head_dim, &t))
        return fail(ATLAS_ERR_RANGE, "sizes overflow");
    if (a->n_new == 0)
        return ok();
    if (!a->k_new || !a->v_new || !a->page_table || !a->start_pos || !a->k_pages || !a->v_pages)
        return fail(ATLAS_ERR_NULL, "k_new, v_new, page_table, start_pos, k_pages and v_pages are required");
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
    if (validate_mode()) {
        const int B = a->batch;
        std::vector<int32_t> sp(B), pt((size_t)B * a->max_pages_per_seq);
        hipError_t e = hipMemcpyAsync(sp.data(), a->start_pos, sizeof(int32_t) * B, hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess)
            e = hipMemcpyAsync(pt.data(), a->page_table, sizeof(int32_t) * pt.size(), hipMemcpyDeviceToHost,
                               stream);
        if (e == hipSuccess)
            e = hipStreamSynchronize(stream);
        if (e != hipSuccess)
            return fail(ATLAS_ERR_DEVICE, "validation copy failed: %s", hipGetErrorString(e));
        const int64_t cap = (int64_t)a->max_pages_per_seq * a->page_size;
        for (int b = 0; b < B; ++b) {
            if (sp[b] < 0 || (int64_t)sp[b] + a->n_new > cap)
                return fail(ATLAS_ERR_RANGE, "start_pos[%d] = %d: positions up to %lld exceed the %lld-token page table",
                            b, sp[b], (long long)sp[b] + a->n_new - 1, (long long)cap);
            for (int64_t p = sp[b]; p < (int64_t)sp[b] + a->n_new; p += a->page_size - (p % a->page_size)) {
                const int32_t id = pt[(size_t)b * a->max_pages_per_seq + p / a->page_size];
                if (id < 0 || id >= a->num_phys_pages)
                    return fail(ATLAS_ERR_POOL, "page_table[%d][%lld] = %d outside the pool of %d pages", b,
                                (long long)(p / a->page_size), id, a->num_phys_pages);
            }
        }
    }
    atlas::AppendArgs k{};
    k.k_new = a->k_new;
    k.v_new = a->v_new;
    k.page_table = a->page_table;
    k.start_pos = a->start_pos;
    k.k_pages = a->k_pages;
    k.v_pages = a->v_pages;
    k.batch = a->batch;
    k.n_new = a->n_new;
    k.hkv = a->num_kv_heads;
    k.row_bytes = a->head_dim * (a->dtype == ATLAS_DTYPE_F32 ? 4 : 2);
    k.page_shift = log2i(a->page_size);
    k.num_phys = a->num_phys_pages;
    k.max_pages = a->max_pages_per_seq;
    hipError_t e = atlas::launch_append(k, stream);
    if (e != hipSuccess)
        return fail(ATLAS_ERR_DEVICE, "append launch: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"

// Host-side page pool: reference counts and a free list under one mutex.
struct atlas_pool {
    std::mutex mu;
    std::vector<int32_t> refs;   // per page; 0 = free
    std::vector<int32_t> free;   // stack of free ids (top = next to hand out)
};

extern "C" {

int32_t atlas_pool_create(int32_t num_pages, atlas_pool **out)
{
    if (!out)
        return fail(ATLAS_ERR_NULL, "out is NULL");
    *out = nullptr;
    if (num_pages < 1)
        return fail(ATLAS_ERR_SHAPE, "num_pages must be >= 1");
    atlas_pool *p = new (std::nothrow) atlas_pool;
    if (!p)
        return fail(ATLAS_ERR_RANGE, "out of host memory");
    p->refs.assign(num_pages, 0);
    p->free.resize(num_pages);
    for (int32_t i = 0; i < num_pages; ++i)
        p->free[i] = num_pages - 1 - i;  // id 0 on top
    *out = p;
    return ok();
}

void atlas_pool_destroy(atlas_pool *pool) { delete pool; }

int32_t atlas_pool_alloc(atlas_pool *pool, int32_t n, int32_t *ids)
{
    if (!pool || (n > 0 && !ids))
        return fail(ATLAS_ERR_NULL, "pool and ids are required");
    if (n < 0)
        return fail(ATLAS_ERR_RANGE, "n must be >= 0");
    std::lock_guard<std::mutex> lock(pool->mu);
    if ((size_t)n > pool->free.size())
        return fail(ATLAS_ERR_POOL, "%d pages requested, %zu free", n, pool->free.size());
    for (int32_t i = 0; i < n; ++i) {
        ids[i] = pool->free.back();
        pool->free.pop_back();
        pool->refs[ids[i]] = 1;
    }
    return ok();
}

int32_t atlas_pool_retain(atlas_pool *pool, int32_t n, const int32_t *ids)
{
    if (!pool || (n > 0 && !ids))
        return fail(ATLAS_ERR_NULL, "pool and ids are required");
    if (n < 0)
        return fail(ATLAS_ERR_RANGE, "n must be >= 0");
    std::lock_guard<std::mutex> lock(pool->mu);
    for (int32_t i = 0; i < n; ++i)
        if (ids[i] < 0 || (size_t)ids[i] >= pool->refs.size() || pool->refs[ids[i]] == 0)
            return fail(ATLAS_ERR_RANGE, "page %d is not in use", ids[i]);
    for (int32_t i = 0; i < n; ++i)
        ++pool->refs[ids[i]];
    return ok();
}

int32_t atlas_pool_release(atlas_pool *pool, int32_t n, const int32_t *ids)
{
    if (!pool || (n > 0 && !ids))
        return fail(ATLAS_ERR_NULL, "pool and ids are required");
    if (n < 0)
        return fail(ATLAS_ERR_RANGE, "n must be >= 0");
    std::lock_guard<std::mutex> lock(pool->mu);
    std::vector<int32_t> drop(pool->refs.size(), 0);
    for (int32_t i = 0; i < n; ++i) {
        if (ids[i] < 0 || (size_t)ids[i] >= pool->refs.size())
            return fail(ATLAS_ERR_RANGE, "page %d outside the pool", ids[i]);
        if (++drop[ids[i]] > pool->refs[ids[i]])
            return fail(ATLAS_ERR_RANGE, "page %d released more often than it is referenced", ids[i]);
    }
    for (int32_t i = 0; i < n; ++i)
        if (--pool->refs[ids[i]] == 0)
            pool->free.push_back(ids[i]);
    return ok();
}

int32_t atlas_pool_free_pages(const atlas_pool *pool)
{
    if (!pool)
        return 0;
    std::lock_guard<std::mutex> lock(const_cast<atlas_pool *>(pool)->mu);
    return (int32_t)pool->free.size();
}

int32_t atlas_pool_refcount(const atlas_pool *pool, int32_t id)
{
    if (!pool)
        return -1;
    std::lock_guard<std::mutex> lock(const_cast<atlas_pool *>(pool)->mu);
    if (id < 0 || (size_t)id >= pool->refs.size())
        return -1;
    return pool->refs[id];
}

}  // extern "C"

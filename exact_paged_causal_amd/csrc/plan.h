// plan.h -- which keys each split-KV work item folds.
//
// Shared by the host planner (grid and workspace sizing) and by the kernels
// (each work item derives its own key span from the device-resident context
// length), and compilable as plain C++ so the CPU tests can check it against
// brute-force enumeration.
//
// A work item covers a set of query rows whose absolute positions lie in
// [pos_min, pos_max].  The keys any of them can see (the union of their
// visible sets; see atlas.h for the visibility rule) are
//   * the window span [lo, pos_max + 1), lo = max(0, pos_min - W + 1) when a
//     window W > 0 is set, else lo = 0, and
//   * the sink tokens [0, min(S, lo)) that fall before the window.
// Both spans are cut at multiples of `split_tokens` (T), so every split
// boundary is a fixed token index independent of where pages live in memory,
// and no split holds more than T keys.  Only pages
// that intersect these spans are ever read (page-granular window skipping,
// ferrox-core kv_swa block alignment idea).  Inside a split each key is still
// masked per row, because rows at different positions see different windows.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define ATLAS_HD __host__ __device__ __forceinline__
#else
#define ATLAS_HD inline
#endif

namespace atlas {

struct SplitPlan {
    int32_t n_splits;   // 0: no row of the item sees any key
    int32_t sink_end;   // sink span [0, sink_end) before the window (0: none)
    int32_t n_sink;     // splits covering the sink span (T-aligned blocks)
    int32_t win_lo;     // window span [win_lo, win_hi)
    int32_t win_hi;
    int32_t first_blk;  // first T-aligned block of the window span
};

ATLAS_HD SplitPlan plan_splits(int32_t pos_min, int32_t pos_max, int32_t window, int32_t sinks,
                               int32_t split_tokens)
{
    SplitPlan p{0, 0, 0, 0, 0, 0};
    if (pos_max < 0)
        return p;
    if (pos_min < 0)
        pos_min = 0;
    const int32_t hi = pos_max + 1;
    int32_t lo = 0;
    if (window > 0) {
        lo = pos_min - window + 1;
        if (lo < 0)
            lo = 0;
        const int32_t s = sinks < lo ? sinks : lo;
        if (s > 0)
            p.sink_end = s;
    }
    p.n_sink = (p.sink_end + split_tokens - 1) / split_tokens;
    p.win_lo = lo;
    p.win_hi = hi;
    p.first_blk = lo / split_tokens;
    const int32_t last_blk = (hi - 1) / split_tokens;
    p.n_splits = p.n_sink + (last_blk - p.first_blk + 1);
    return p;
}

// Key range [*a, *b) of split s (0 <= s < n_splits).
ATLAS_HD void split_range(const SplitPlan &p, int32_t s, int32_t split_tokens, int32_t *a,
                          int32_t *b)
{
    if (s < p.n_sink) {
        *a = s * split_tokens;
        const int32_t e = *a + split_tokens;
        *b = e < p.sink_end ? e : p.sink_end;
        return;
    }
    s -= p.n_sink;
    const int32_t lo = (p.first_blk + s) * split_tokens;
    const int32_t hi = lo + split_tokens;
    *a = lo > p.win_lo ? lo : p.win_lo;
    *b = hi < p.win_hi ? hi : p.win_hi;
}

// Upper bound of n_splits over every context length <= max_context: the sink
// blocks cover [0, lo) and the window blocks [lo, hi), so together they take
// at most one block more than ceil(hi / T).
ATLAS_HD int32_t max_splits_bound(int32_t max_context, int32_t split_tokens, bool with_sinks)
{
    return (max_context + split_tokens - 1) / split_tokens + (with_sinks ? 1 : 0);
}

// Rows of K/V head g: every (query i, member j of g's q-head group), ordered
// r = i * group_size + j; a row chunk is `rows_per_item` consecutive rows.
// Query i sits at position context - q_len + i.
struct ChunkRows {
    int32_t r0, r1;          // rows [r0, r1) of the chunk (r0 >= r1: empty)
    int32_t pos_min, pos_max;
};

ATLAS_HD ChunkRows chunk_rows(int32_t chunk, int32_t rows_per_item, int32_t group_size,
                              int32_t q_len, int32_t context)
{
    ChunkRows c;
    const int32_t n_rows = q_len * group_size;
    c.r0 = chunk * rows_per_item;
    c.r1 = c.r0 + rows_per_item < n_rows ? c.r0 + rows_per_item : n_rows;
    if (c.r0 >= c.r1) {
        c.pos_min = c.pos_max = -1;
        return c;
    }
    c.pos_min = context - q_len + c.r0 / group_size;
    c.pos_max = context - q_len + (c.r1 - 1) / group_size;
    return c;
}

// Key blocks of `block` keys a tiled query block visits (rows at positions
// [pos_lo, pos_hi], last key any of them can see key_hi): with a window W the
// blocks holding sink keys below the first window block, then the blocks from
// the one holding pos_lo - W + 1 up to key_hi's; without one every block up
// to key_hi's.  Visit index c maps to block c (c < n_sink) or
// first_win + c - n_sink.
struct TiledBlocks {
    int32_t n;          // blocks visited (0: none)
    int32_t n_sink;
    int32_t first_win;
};

ATLAS_HD TiledBlocks tiled_blocks(int32_t pos_lo, int32_t key_hi, int32_t window, int32_t sinks, int32_t block)
{
    TiledBlocks t{0, 0, 0};
    const int32_t kb_last = key_hi >= 0 ? key_hi / block : -1;
    if (kb_last < 0)
        return t;
    if (window > 0) {
        const int32_t lo_key = pos_lo - window + 1;
        t.first_win = lo_key > 0 ? lo_key / block : 0;
        const int32_t sb = (sinks + block - 1) / block;
        t.n_sink = sinks > 0 ? (sb < t.first_win ? sb : t.first_win) : 0;
    }
    t.n = t.n_sink + (kb_last - t.first_win + 1);
    return t;
}

ATLAS_HD int32_t tiled_block_at(const TiledBlocks &t, int32_t c)
{
    return c < t.n_sink ? c : t.first_win + (c - t.n_sink);
}

}  // namespace atlas

// Host build of the library's split planner (exact_paged_causal_amd/csrc/plan.h)
// with C entry points, so the CPU tests can check it against brute force.
#include "plan.h"

extern "C" {
void probe_plan(int pos_min, int pos_max, int window, int sinks, int split_tokens, int *out6)
{
    atlas::SplitPlan p = atlas::plan_splits(pos_min, pos_max, window, sinks, split_tokens);
    out6[0] = p.n_splits;
    out6[1] = p.sink_end;
    out6[2] = p.n_sink;
    out6[3] = p.win_lo;
    out6[4] = p.win_hi;
    out6[5] = p.first_blk;
}

void probe_ranges(int pos_min, int pos_max, int window, int sinks, int split_tokens, int *ranges,
                  int cap, int *n_out)
{
    atlas::SplitPlan p = atlas::plan_splits(pos_min, pos_max, window, sinks, split_tokens);
    int n = p.n_splits < cap ? p.n_splits : cap;
    for (int s = 0; s < n; ++s)
        atlas::split_range(p, s, split_tokens, &ranges[2 * s], &ranges[2 * s + 1]);
    *n_out = p.n_splits;
}

int probe_bound(int max_context, int split_tokens, int with_sinks)
{
    return atlas::max_splits_bound(max_context, split_tokens, with_sinks != 0);
}

void probe_chunk(int chunk, int rows_per_item, int group_size, int q_len, int context, int *out4)
{
    atlas::ChunkRows c = atlas::chunk_rows(chunk, rows_per_item, group_size, q_len, context);
    out4[0] = c.r0;
    out4[1] = c.r1;
    out4[2] = c.pos_min;
    out4[3] = c.pos_max;
}

void probe_tiled(int pos_lo, int key_hi, int window, int sinks, int block, int *blocks, int cap, int *n_out)
{
    atlas::TiledBlocks t = atlas::tiled_blocks(pos_lo, key_hi, window, sinks, block);
    int n = t.n < cap ? t.n : cap;
    for (int c = 0; c < n; ++c)
        blocks[c] = atlas::tiled_block_at(t, c);
    *n_out = t.n;
}
}

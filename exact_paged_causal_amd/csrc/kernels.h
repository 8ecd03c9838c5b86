// kernels.h -- internal interface between the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace atlas {

constexpr int kMaxHeads = 256;

// q-head <-> K/V-head grouping, built on the host from head_map and passed by
// value in the kernel arguments (constant for the whole launch).
struct HeadGroups {
    int16_t start[kMaxHeads + 1];  // q-heads of K/V head g: list[start[g] .. start[g+1])
    int16_t list[kMaxHeads];
    int16_t group_of[kMaxHeads];   // q-head -> K/V head
    int16_t slot_of[kMaxHeads];    // q-head -> its index inside the group
    int32_t max_group;             // largest group size
    int32_t pad;
};

// Score and mask modifications of atlas_attend_mods.  any = 0 selects the
// plain causal kernels; otherwise key j of a row at position pos of sequence
// b (query i) is visible when (causal ? j <= pos : j < context) and, with a
// mask, bit j of mask row (b, i) is set; the logit gains -alibi[h] |pos - j|
// after the softcap.
struct Mods {
    const float *alibi;         // [hq] slopes or null
    const uint32_t *mask;       // [B][q_len][mask_words] bits or null
    int32_t mask_words;
    int32_t causal;
    int32_t any;
    int32_t pad;
};

// Everything a split-KV work item and the merge pass need.
struct SplitArgs {
    const void *q;
    const void *k_pages;
    const void *v_pages;
    const int32_t *page_table;
    const int32_t *context_lens;
    const int32_t *window;      // may be null
    const int32_t *sinks;       // may be null
    const float *softcap;       // may be null
    float *ws_acc;              // [rows][max_splits][D]  unnormalised accumulators
    float *ws_ml;               // [rows][max_splits][2]  (running max in log2 units, sum)
    float *out;                 // [B][q_len][Hq][D]
    float *lse;                 // [B][q_len][Hq] or null
    int32_t batch, q_len, hq, hkv, head_dim;
    int32_t page_shift;         // log2(page_size)
    int32_t num_phys, max_pages, max_context;
    int32_t split_tokens, max_splits;
    int32_t rows_per_item;      // rows of one work item (a chunk of a K/V head's rows)
    int32_t n_chunks;           // chunks per K/V head
    float scale;
    // In-kernel regeneration: page-table entries of -1 are regenerated from
    // (regen_seed, regen_layer, sequence key, logical page); the key of
    // sequence b is seq_keys[b] (clamped into [0, 65536)), or b without them.
    uint64_t regen_seed;
    const int32_t *seq_keys;    // may be null
    int32_t regen_layer;
    int32_t regen;              // 0: every page is read from the arenas
    // bf16 K/V fold only: q is fp32 (split into bf16 high and low parts).
    int32_t q_f32;
    int32_t pad0;
    // Merge of the tiled prefill's key splits (tiled_blocks > 0): the splits
    // of query i are ceil(n / tiled_blocks) for the n key blocks its query
    // block of tiled_npos positions visits (plan.h tiled_blocks).
    int32_t tiled_blocks;
    int32_t tiled_npos;
    Mods mods;
    HeadGroups groups;
};

struct RegenArgs {
    uint64_t seed;
    const int32_t *jobs;        // [n_jobs][3] (seq, logical page, physical page)
    void *k_pages;
    void *v_pages;
    int32_t layer, hkv, head_dim, page_shift, num_phys, n_jobs;
};

// Largest page-id list one split work item stages in LDS.
constexpr int kMaxSplitPages = 2048;
// Most splits one output row may have (the merge keeps their weights in LDS).
constexpr int kMaxMergeSplits = 8192;

hipError_t launch_split_valu(const SplitArgs &a, hipStream_t stream);   // fp32 K/V
hipError_t launch_split_mfma(const SplitArgs &a, hipStream_t stream);   // bf16 K/V
hipError_t launch_merge(const SplitArgs &a, hipStream_t stream);
hipError_t launch_regen(const RegenArgs &a, int dtype, hipStream_t stream);

struct AppendArgs {
    const void *k_new;          // [B][n_new][Hkv][row_bytes]
    const void *v_new;
    const int32_t *page_table;
    const int32_t *start_pos;
    void *k_pages;
    void *v_pages;
    int32_t batch, n_new, hkv, row_bytes, page_shift, num_phys, max_pages;
};

hipError_t launch_append(const AppendArgs &a, hipStream_t stream);

struct PrefillArgs {
    const void *q;
    const void *k_pages;
    const void *v_pages;
    const int32_t *page_table;
    const int32_t *context_lens;
    const int32_t *window;      // may be null
    const int32_t *sinks;       // may be null
    const float *softcap;       // may be null
    float *out;
    float *lse;
    int32_t batch, q_len, hq, hkv, head_dim, page_shift, num_phys, max_pages, max_context;
    int32_t n_qblocks;          // query blocks per (sequence, K/V head)
    float scale;
    // Key splits (split_blocks > 0): workgroup (query block, split s) visits
    // blocks [s * split_blocks, (s + 1) * split_blocks) of the block list and
    // writes unnormalised partial states for the merge (SplitArgs layout).
    int32_t split_blocks;
    int32_t max_splits;
    float *ws_acc;              // [rows][max_splits][D]
    float *ws_ml;               // [rows][max_splits][2]
    Mods mods;
    HeadGroups groups;
};

hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t stream);   // bf16 Q/K/V
hipError_t launch_prefill_split(const PrefillArgs &a, hipStream_t stream);  // fp32 Q/K/V, split fp16 operands

// Validation-mode NaN/Inf scan of q and the K/V rows each context covers.
struct ScanArgs {
    const void *q;
    const void *k_pages;
    const void *v_pages;
    const int32_t *page_table;
    const int32_t *context_lens;
    int *flag;                  // bit 0: NaN/Inf; bit 1: beyond the fp16 range (cleared by the caller)
    int32_t batch, q_len, hq, hkv, head_dim, page_shift, num_phys, max_pages, max_context;
    int32_t check_f16;          // 1: flag V values beyond 65504 (the tiled prefills' fp16 P.V products)
};

hipError_t launch_scan(const ScanArgs &a, int q_dtype, int kv_dtype, hipStream_t stream);

}  // namespace atlas

// cache.cpp -- byte-bounded hot-page cache: which K/V pages stay resident.
//
// CFR-Atlas README: the runtime keeps selected pages in a byte-bounded hot
// cache and regenerates cold pages; the library owns the cache, eviction and
// accounting, the caller picks the budget and the admission policy
// (Config::hot_cache_bytes, admit_regenerated_pages, the KeepRecent policy),
// and admission changes latency and residency only, never the attention
// result ("Core contract").
//
// Here the resident pages live in a hot pool of physical pages (ids 0 ..
// capacity - 1, capacity = hot_cache_bytes / page_bytes); a page not in the
// pool is regenerated inside the attention kernel (page-table entry
// ATLAS_PAGE_REGENERATE), so cold pages need no scratch memory at all.  One
// planning call per attention call (one layer, a batch of sequences):
//   1. the call's resident pages are hits and are stamped with the call's
//      clock;
//   2. KeepRecent: the pages holding any of a sequence's last recent_tokens
//      tokens are admitted first (newest first), taking a free slot or
//      evicting the least recently used page this call does not read
//      (pages outside any recent window before those inside one);
//   3. admit_regenerated: the call's other cold pages take the slots still
//      free, in (sequence, page) order, without evicting;
//   4. the page table maps every page to its slot or to
//      ATLAS_PAGE_REGENERATE; every admission is a regeneration job
//      (sequence id, logical page, slot) for atlas_regenerate_pages, to run
//      before the attention call.
// A sequence id is also the sequence's generator key (the regenerator and
// the in-kernel regeneration take the same key), so a resident page holds
// the same values whichever batch row the sequence occupies in a later call;
// ids are therefore limited to the generator's 16-bit key range.
// All checks run before any state changes (transactional accounting).
#include <algorithm>
#include <cstdint>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "../../include/atlas.h"
#include "status.h"

namespace {

struct Key {
    int64_t seq;
    int32_t layer;
    int32_t page;
    bool operator==(const Key &o) const { return seq == o.seq && layer == o.layer && page == o.page; }
};

struct KeyHash {
    size_t operator()(const Key &k) const
    {
        uint64_t h = (uint64_t)k.seq * 0x9E3779B97F4A7C15ull;
        h ^= ((uint64_t)(uint32_t)k.layer << 32 | (uint32_t)k.page) + 0x7F4A7C159E3779B9ull + (h << 6) + (h >> 2);
        return (size_t)h;
    }
};

struct Entry {
    int32_t slot;
    bool pinned;        // inside its sequence's recent window when last planned
    uint64_t last_use;  // clock of the last call that read it
};

}  // namespace

struct atlas_cache {
    std::mutex mu;
    atlas_cache_config cfg;
    int32_t capacity = 0;
    uint64_t clock = 0;
    std::vector<int32_t> free_slots;  // stack, lowest ids on top
    std::vector<Key> slot_key;        // slot -> page (valid while resident)
    std::unordered_map<Key, Entry, KeyHash> map;
    atlas_cache_stats stats{};
};

using atlas::fail;
using atlas::ok;

extern "C" {

int32_t atlas_cache_create(const atlas_cache_config *cfg, atlas_cache **out)
{
    if (!cfg || !out)
        return fail(ATLAS_ERR_NULL, "cfg and out are required");
    *out = nullptr;
    if (cfg->page_bytes < 1 || cfg->page_size < 1 || cfg->hot_cache_bytes < 0 || cfg->recent_tokens < 0)
        return fail(ATLAS_ERR_SHAPE, "page_bytes and page_size must be >= 1, hot_cache_bytes and recent_tokens >= 0");
    if (cfg->admit_regenerated != 0 && cfg->admit_regenerated != 1)
        return fail(ATLAS_ERR_RANGE, "admit_regenerated must be 0 or 1");
    const int64_t cap = cfg->hot_cache_bytes / cfg->page_bytes;
    if (cap > (1 << 24))
        return fail(ATLAS_ERR_RANGE, "hot cache of %lld pages exceeds 2^24", (long long)cap);
    atlas_cache *c = new atlas_cache();
    c->cfg = *cfg;
    c->capacity = (int32_t)cap;
    c->free_slots.resize(cap);
    for (int64_t i = 0; i < cap; ++i)
        c->free_slots[i] = (int32_t)(cap - 1 - i);
    c->slot_key.resize(cap);
    c->stats.capacity_pages = cap;
    *out = c;
    return ok();
}

void atlas_cache_destroy(atlas_cache *c) { delete c; }

int32_t atlas_cache_plan(atlas_cache *c, int32_t layer, int32_t batch, const int64_t *seq_ids,
                         const int32_t *context_lens, int32_t max_pages_per_seq, int32_t *page_table,
                         int32_t *admit_jobs, int32_t max_jobs, int32_t *n_jobs, int32_t *n_cold)
{
    if (!c || !seq_ids || !context_lens || !page_table || !n_jobs || (max_jobs > 0 && !admit_jobs))
        return fail(ATLAS_ERR_NULL, "cache, seq_ids, context_lens, page_table and n_jobs are required");
    if (batch < 1 || max_pages_per_seq < 1 || max_jobs < 0 || layer < 0)
        return fail(ATLAS_ERR_SHAPE, "batch and max_pages_per_seq must be >= 1, layer and max_jobs >= 0");
    std::lock_guard<std::mutex> lock(c->mu);
    const int P = c->cfg.page_size;
    const int64_t max_ctx = (int64_t)max_pages_per_seq * P;
    int64_t total_pages = 0;
    for (int b = 0; b < batch; ++b) {
        if (context_lens[b] < 1 || context_lens[b] > max_ctx)
            return fail(ATLAS_ERR_RANGE, "context_lens[%d] = %d outside [1, %lld]", b, context_lens[b],
                        (long long)max_ctx);
        if (seq_ids[b] < 0 || seq_ids[b] >= 65536)
            return fail(ATLAS_ERR_RANGE, "seq_ids[%d] = %lld: sequence ids key the generator and must lie in "
                                         "[0, 65536)", b, (long long)seq_ids[b]);
        for (int b2 = 0; b2 < b; ++b2)
            if (seq_ids[b2] == seq_ids[b])
                return fail(ATLAS_ERR_SHAPE, "sequence id %lld appears twice in one call", (long long)seq_ids[b]);
        total_pages += (context_lens[b] + P - 1) / P;
    }
    const int64_t most_jobs = std::min<int64_t>(total_pages, c->capacity);
    if (max_jobs < most_jobs)
        return fail(ATLAS_ERR_SHAPE, "max_jobs %d < %lld (admissions are bounded by the call's pages and the "
                                     "cache capacity)", max_jobs, (long long)most_jobs);

    const uint64_t now = ++c->clock;
    // 1. hits
    int64_t hits = 0;
    for (int b = 0; b < batch; ++b) {
        const int np = (context_lens[b] + P - 1) / P;
        const int first_recent = c->cfg.recent_tokens > 0
                                     ? (int)(std::max<int64_t>(0, (int64_t)context_lens[b] - c->cfg.recent_tokens) / P)
                                     : np;
        for (int lp = 0; lp < np; ++lp) {
            auto it = c->map.find(Key{seq_ids[b], layer, lp});
            if (it != c->map.end()) {
                it->second.last_use = now;
                it->second.pinned = lp >= first_recent;
                ++hits;
            }
        }
    }
    int32_t jobs = 0;
    int64_t evicted = 0;
    auto admit = [&](int b, int lp, bool pinned, bool may_evict) -> bool {
        int32_t slot;
        if (!c->free_slots.empty()) {
            slot = c->free_slots.back();
            c->free_slots.pop_back();
        } else {
            if (!may_evict)
                return false;
            // Least recently used page this call does not read; pages outside
            // a recent window first.
            int32_t victim = -1;
            bool v_pinned = true;
            uint64_t v_use = UINT64_MAX;
            for (int32_t s = 0; s < c->capacity; ++s) {
                const Entry &e = c->map.at(c->slot_key[s]);
                if (e.last_use == now)
                    continue;
                if ((!e.pinned && v_pinned) || (e.pinned == v_pinned && e.last_use < v_use)) {
                    victim = s;
                    v_pinned = e.pinned;
                    v_use = e.last_use;
                }
            }
            if (victim < 0)
                return false;
            c->map.erase(c->slot_key[victim]);
            slot = victim;
            ++evicted;
        }
        const Key k{seq_ids[b], layer, lp};
        c->slot_key[slot] = k;
        c->map[k] = Entry{slot, pinned, now};
        admit_jobs[3 * jobs + 0] = (int32_t)seq_ids[b];
        admit_jobs[3 * jobs + 1] = lp;
        admit_jobs[3 * jobs + 2] = slot;
        ++jobs;
        return true;
    };
    // 2. KeepRecent, newest pages first
    if (c->cfg.recent_tokens > 0 && c->capacity > 0) {
        for (int b = 0; b < batch; ++b) {
            const int np = (context_lens[b] + P - 1) / P;
            const int first_recent =
                (int)(std::max<int64_t>(0, (int64_t)context_lens[b] - c->cfg.recent_tokens) / P);
            for (int lp = np - 1; lp >= first_recent; --lp)
                if (c->map.find(Key{seq_ids[b], layer, lp}) == c->map.end())
                    admit(b, lp, true, true);
        }
    }
    // 3. admit the call's other cold pages into free slots
    if (c->cfg.admit_regenerated) {
        for (int b = 0; b < batch && !c->free_slots.empty(); ++b) {
            const int np = (context_lens[b] + P - 1) / P;
            for (int lp = 0; lp < np && !c->free_slots.empty(); ++lp)
                if (c->map.find(Key{seq_ids[b], layer, lp}) == c->map.end())
                    admit(b, lp, false, false);
        }
    }
    // 4. page table
    int64_t misses = 0;
    for (int b = 0; b < batch; ++b) {
        const int np = (context_lens[b] + P - 1) / P;
        for (int lp = 0; lp < max_pages_per_seq; ++lp) {
            int32_t v = ATLAS_PAGE_REGENERATE;
            if (lp < np) {
                auto it = c->map.find(Key{seq_ids[b], layer, lp});
                if (it != c->map.end())
                    v = it->second.slot;
                else
                    ++misses;
            }
            page_table[(int64_t)b * max_pages_per_seq + lp] = v;
        }
    }
    *n_jobs = jobs;
    if (n_cold)
        *n_cold = (int32_t)misses;
    c->stats.hits += hits;
    c->stats.misses += misses;
    c->stats.admitted += jobs;
    c->stats.evicted += evicted;
    c->stats.resident_pages = (int64_t)c->map.size();
    c->stats.resident_bytes = c->stats.resident_pages * c->cfg.page_bytes;
    return ok();
}

int32_t atlas_cache_drop_sequence(atlas_cache *c, int64_t seq_id)
{
    if (!c)
        return fail(ATLAS_ERR_NULL, "cache is NULL");
    std::lock_guard<std::mutex> lock(c->mu);
    std::vector<int32_t> freed;
    for (auto it = c->map.begin(); it != c->map.end();) {
        if (it->first.seq == seq_id) {
            freed.push_back(it->second.slot);
            it = c->map.erase(it);
        } else {
            ++it;
        }
    }
    // keep the lowest ids on top of the free stack
    c->free_slots.insert(c->free_slots.end(), freed.begin(), freed.end());
    std::sort(c->free_slots.begin(), c->free_slots.end(), std::greater<int32_t>());
    c->stats.resident_pages = (int64_t)c->map.size();
    c->stats.resident_bytes = c->stats.resident_pages * c->cfg.page_bytes;
    return ok();
}

int32_t atlas_cache_get_stats(atlas_cache *c, atlas_cache_stats *out)
{
    if (!c || !out)
        return fail(ATLAS_ERR_NULL, "cache and out are required");
    std::lock_guard<std::mutex> lock(c->mu);
    *out = c->stats;
    return ok();
}

}  // extern "C"

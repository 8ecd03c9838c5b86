"""Host tests of the byte-bounded hot-page cache (atlas_cache_*): the budget
bound, KeepRecent priority, least-recently-used eviction of pages a call
does not read, admission of regenerated pages into free slots only, the page
table / job contract and transactional errors.  No GPU needed."""
import numpy as np
import pytest

import exact_paged_causal_amd as atlas

P = 16


def cache(slots, recent=0, admit=True):
    return atlas.HotCache(slots * 1000, 1000, P, recent_tokens=recent, admit_regenerated=admit)


def resident(pt):
    return {(b, lp): int(s) for b in range(pt.shape[0]) for lp, s in enumerate(pt[b]) if s >= 0}


def check_contract(pt, jobs, ctx, slots, ids):
    """Slots are distinct, inside the pool; entries past the context are
    REGENERATE; every job (sequence id, logical page, slot) admits a page the
    table now maps to its slot in that sequence's batch row."""
    res = resident(pt)
    assert len(set(res.values())) == len(res) and all(0 <= s < slots for s in res.values())
    for b, L in enumerate(ctx):
        np_ = (L + P - 1) // P
        assert (pt[b, np_:] == atlas.ATLAS_PAGE_REGENERATE).all()
    for sid, lp, s in jobs:
        assert pt[list(ids).index(sid), lp] == s


def test_budget_and_admission_order():
    c = cache(6, recent=32)
    ctx = [50, 20]                      # 4 + 2 pages
    pt, jobs = c.plan(0, [7, 9], ctx, 4)
    check_contract(pt, jobs, ctx, 6, [7, 9])
    # recent pages first (newest first per sequence), then the rest while slots
    # last; jobs name the sequence by its id (its generator key)
    assert [tuple(j[:2]) for j in jobs] == [(7, 3), (7, 2), (7, 1), (9, 1), (9, 0), (7, 0)]
    st = c.stats()
    assert st["resident_pages"] == 6 and st["resident_bytes"] == 6000 and st["admitted"] == 6
    # the same call again: all hits, nothing admitted
    assert c.last_cold == 0                       # every page of the call admitted
    pt2, jobs2 = c.plan(0, [7, 9], ctx, 4)
    assert len(jobs2) == 0 and np.array_equal(pt, pt2)
    assert c.stats()["hits"] == 6 and c.stats()["misses"] == 0
    # the sequences swap batch rows: the same pages hit, in the other rows
    pt3, jobs3 = c.plan(0, [9, 7], ctx[::-1], 4)
    assert len(jobs3) == 0 and np.array_equal(pt3, pt[::-1])


def test_no_admission_without_policy_leaves_pages_cold():
    c = cache(4, recent=0, admit=False)
    pt, jobs = c.plan(0, [1], [40], 3)
    assert len(jobs) == 0 and (pt == atlas.ATLAS_PAGE_REGENERATE).all()
    assert c.last_cold == 3
    assert c.stats()["misses"] == 3 and c.stats()["resident_pages"] == 0


def test_admit_regenerated_never_evicts():
    c = cache(2, recent=0, admit=True)
    pt, jobs = c.plan(0, [1], [64], 4)            # 4 pages, 2 slots: pages 0 and 1 admitted
    assert [tuple(j[:2]) for j in jobs] == [(1, 0), (1, 1)]
    pt, jobs = c.plan(0, [2], [64], 4)            # another sequence: no free slot, no eviction
    assert len(jobs) == 0 and (pt == atlas.ATLAS_PAGE_REGENERATE).all()
    assert c.stats()["evicted"] == 0


def test_recent_pages_evict_the_least_recently_used_unpinned_page():
    c = cache(3, recent=16, admit=True)
    c.plan(0, [1], [48], 3)                       # seq 1: page 2 pinned, pages 0, 1 admitted too
    c.plan(0, [2], [16], 1)                       # seq 2 page 0 (pinned): evicts seq 1's LRU unpinned page
    st = c.stats()
    assert st["evicted"] == 1 and st["resident_pages"] == 3
    pt, jobs = c.plan(0, [1], [48], 3)
    # seq 1's pinned page 2 survived; one of its older pages was evicted and stays cold
    assert pt[0, 2] >= 0 and int((pt[0] < 0).sum()) == 1 and len(jobs) == 0


def test_pages_read_by_the_call_are_never_evicted():
    c = cache(2, recent=64, admit=False)
    pt, jobs = c.plan(0, [5], [64], 4)            # 4 recent pages, 2 slots: the two newest
    assert sorted(int(j[1]) for j in jobs) == [2, 3]
    assert (pt[0, :2] == atlas.ATLAS_PAGE_REGENERATE).all() and c.stats()["evicted"] == 0


def test_layers_and_drop_sequence():
    c = cache(8, recent=0, admit=True)
    pt0, j0 = c.plan(0, [3], [32], 2)
    pt1, j1 = c.plan(1, [3], [32], 2)             # another layer: its own pages
    assert len(j0) == 2 and len(j1) == 2 and set(pt0[0]).isdisjoint(set(pt1[0]))
    c.drop_sequence(3)
    assert c.stats()["resident_pages"] == 0
    pt, j = c.plan(0, [4], [64], 4)
    assert sorted(int(s) for s in pt[0]) == [0, 1, 2, 3]   # freed slots are reused, lowest first


def test_errors_change_nothing():
    c = cache(4, recent=16)
    with pytest.raises(atlas.AtlasError) as ei:
        c.plan(0, [1, 1], [10, 10], 2)            # duplicate sequence id
    assert ei.value.status == atlas.ATLAS_ERR_SHAPE
    with pytest.raises(atlas.AtlasError) as ei:
        c.plan(0, [1], [100], 2)                  # context beyond the table
    assert ei.value.status == atlas.ATLAS_ERR_RANGE
    with pytest.raises(atlas.AtlasError) as ei:
        c.plan(0, [1], [0], 2)
    assert ei.value.status == atlas.ATLAS_ERR_RANGE
    for bad_id in (-1, 65536):                     # ids key the generator: 16 bits
        with pytest.raises(atlas.AtlasError) as ei:
            c.plan(0, [2, bad_id], [10, 10], 2)
        assert ei.value.status == atlas.ATLAS_ERR_RANGE
    assert c.stats() == {"capacity_pages": 4, "resident_pages": 0, "resident_bytes": 0, "hits": 0, "misses": 0,
                         "admitted": 0, "evicted": 0}
    with pytest.raises(atlas.AtlasError) as ei:
        atlas.HotCache(100, 0, 16)
    assert ei.value.status == atlas.ATLAS_ERR_SHAPE


def test_random_traffic_respects_the_budget():
    rng = np.random.default_rng(3)
    slots = 20
    c = cache(slots, recent=24, admit=True)
    lens = {s: int(rng.integers(1, 200)) for s in range(6)}
    for step in range(60):
        ids = sorted(rng.choice(6, size=int(rng.integers(1, 4)), replace=False).tolist())
        for s in ids:
            lens[s] += int(rng.integers(0, 3))
        ctx = [lens[s] for s in ids]
        pt, jobs = c.plan(int(rng.integers(0, 2)), ids, ctx, 16)
        check_contract(pt, jobs, ctx, slots, ids)
        assert c.stats()["resident_pages"] <= slots
        if step % 17 == 16:
            c.drop_sequence(int(rng.integers(0, 6)))

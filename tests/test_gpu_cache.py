"""GPU test of the hot-page cache in the decode path: each call plans
residency (atlas_cache_plan), regenerates the admitted pages into their hot
slots (atlas_regenerate_pages) and decodes with the remaining cold pages
generated in the kernel (atlas_attend_decode_regen).  CFR-Atlas "Core
contract": admission changes residency and latency only, so the output must
be bit-identical to decoding with every page generated in the kernel, for
every budget and policy, as the cache warms up and the contexts grow.  The
oracle checks the reference once.  Each test prints its case first."""
import math

import numpy as np
import pytest
import torch

import harness as H
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_paged_causal_amd  # noqa: F401  (fails loudly if libatlas.so is missing)
    yield


def say(*a):
    print(*a, flush=True)


B, HQ, HKV, D, P, MAXP = 3, 8, 2, 64, 64, 64
PAGE_BYTES = HKV * P * D * 4 * 2
SEED, LAYER = 11, 3


def decode_all_cold(q, ctx, keys):
    import exact_paged_causal_amd as atlas
    k = torch.zeros((1, HKV, P, D), device="cuda")
    pt = torch.full((B, MAXP), atlas.ATLAS_PAGE_REGENERATE, dtype=torch.int32, device="cuda")
    return atlas.atlas_attend_decode_regen(q, k, torch.zeros_like(k), pt, ctx, 1.0 / math.sqrt(D), seed=SEED,
                                           layer=LAYER, seq_keys=keys)


@pytest.mark.parametrize("slots,recent,admit", [
    (0, 0, True), (7, 256, False), (7, 256, True), (40, 0, True), (400, 1024, True),
], ids=lambda x: str(x))
def test_cached_decode_is_bit_identical(slots, recent, admit):
    import exact_paged_causal_amd as atlas
    say(f"[cache] slots={slots} recent={recent} admit={admit}")
    cache = atlas.HotCache(slots * PAGE_BYTES, PAGE_BYTES, P, recent_tokens=recent, admit_regenerated=admit)
    k = torch.full((max(slots, 1), HKV, P, D), float("nan"), device="cuda")   # unwritten slots are never read
    v = torch.full_like(k, float("nan"))
    lens_of = {101: 3000, 202: 1500, 303: 800}
    # the sequences change batch rows from step to step (a serving loop
    # reorders its batch); a sequence's id is its generator key
    orders = [[101, 202, 303], [303, 101, 202], [202, 303, 101], [101, 303, 202]]
    for step in range(4):
        if step == 2:
            lens_of = {s: L + 70 for s, L in lens_of.items()}   # the contexts grow into new pages
        seq_ids = orders[step]
        lens = np.array([lens_of[s] for s in seq_ids], np.int32)
        ctx = torch.from_numpy(lens).cuda()
        keys = torch.tensor(seq_ids, dtype=torch.int32, device="cuda")
        q = workloads.randn((B, 1, HQ, D), seed=500 + step, device="cuda")
        ref_o, ref_l = decode_all_cold(q, ctx, keys)
        pt, jobs = cache.plan(LAYER, seq_ids, lens, MAXP)
        if len(jobs):
            atlas.atlas_regenerate_pages(k, v, torch.from_numpy(jobs).cuda(), seed=SEED, layer=LAYER)
        out, lse = atlas.atlas_attend_decode_regen(q, k, v, torch.from_numpy(pt).cuda(), ctx, 1.0 / math.sqrt(D),
                                                   seed=SEED, layer=LAYER, seq_keys=keys)
        torch.cuda.synchronize()
        st = cache.stats()
        say(f"[cache] step {step}: {len(jobs)} admitted, stats {st}")
        assert st["resident_pages"] <= slots
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"step {step}"
        if cache.last_cold == 0:
            # every page resident: the plain decode over the same table gives the same bits
            o2, l2 = atlas.atlas_attend_decode(q, k, v, torch.from_numpy(pt).cuda(), ctx, 1.0 / math.sqrt(D))
            torch.cuda.synchronize()
            assert torch.equal(o2, ref_o) and torch.equal(l2, ref_l), f"plain decode, step {step}"
    if slots >= 400:
        assert st["misses"] == 0 or step < 1
        assert st["hits"] > 0


def test_reference_matches_oracle():
    """The all-cold reference itself against the oracle (the regenerated
    workload's rows come from the oracle's own generator)."""
    w = workloads.Workload("cache_ref", seed=SEED, batch=B, hq=HQ, hkv=HKV, head_dim=D, page_size=P, dtype="f32",
                           q_len=1, context_lens=np.array([3000, 1500, 800], np.int32), scale=1.0 / math.sqrt(D),
                           regenerated=True, hot_fraction=0.0, shuffle_pages=True,
                           seq_keys=np.array([303, 101, 202], np.int32))
    w.layer = LAYER
    say("[cache] reference vs oracle")
    inp = H.build(w)
    out, lse = decode_all_cold(inp.q, inp.context_lens, H.seq_keys_tensor(w))
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what="all-cold reference")

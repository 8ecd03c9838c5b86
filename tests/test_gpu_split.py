"""GPU parity of the regenerator and the split-KV path (decode and short
prefill) against the fp64 oracle, through the C ABI.

Each test prints the case it runs before touching the GPU."""
import math
import os

import numpy as np
import pytest
import torch

import harness as H
import oracle
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


def small(name="custom", *, batch=1, hq=4, hkv=1, d=64, page=16, dtype="f32", q_len=1, lens=(37,),
          scale=None, regenerated=False, hot=1.0, shuffle=True, window=None, sinks=None, softcap=None,
          seed=11, q_dtype=None):
    lens = np.asarray(lens, np.int32)
    return workloads.Workload(
        name, seed=seed, batch=batch, hq=hq, hkv=hkv, head_dim=d, page_size=page, dtype=dtype,
        q_len=q_len, context_lens=lens, scale=(1.0 / math.sqrt(d)) if scale is None else scale,
        regenerated=regenerated, hot_fraction=hot, shuffle_pages=shuffle, q_dtype=q_dtype,
        window=None if window is None else np.asarray(window, np.int32),
        sinks=None if sinks is None else np.asarray(sinks, np.int32),
        softcap=None if softcap is None else np.asarray(softcap, np.float32))


# ---------------------------------------------------------------- regen

@pytest.mark.parametrize("dtype,d,page", [("f32", 64, 16), ("f32", 128, 1), ("bf16", 128, 64),
                                          ("bf16", 64, 512)])
def test_regen_matches_oracle_generator(dtype, d, page):
    """Every regenerated element against the oracle's fp64 value: fp32 within
    1e-6 (1 + |z|); bf16 within half a bf16 ulp of it plus the same slack."""
    import exact_paged_causal_amd as atlas
    say(f"[regen] dtype={dtype} D={d} P={page}")
    hkv, num_phys, seed, layer = 3, 5, 0xABCDEF0123, 7
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    k = torch.full((num_phys, hkv, page, d), 123.0, dtype=dt, device="cuda")
    v = torch.full_like(k, 123.0)
    jobs_np = np.array([[0, 0, 3], [5, 2, 0], [1, 7, 4], [2, 1, 99], [3, 1, -1]], np.int32)
    atlas.atlas_regenerate_pages(k, v, torch.from_numpy(jobs_np).cuda(), seed=seed, layer=layer)
    kh, vh = k.float().cpu().numpy(), v.float().cpu().numpy()
    for seq, lp, phys in jobs_np[:3]:
        for h in range(hkv):
            for tensor, arena in ((oracle.TENSOR_K, kh), (oracle.TENSOR_V, vh)):
                z = oracle.regen_rows(seed, layer, int(seq), tensor, h, int(lp) * page, page, d, "f64")
                got = arena[phys, h].astype(np.float64)
                bound = 1e-6 * (1 + np.abs(z))
                if dtype == "bf16":
                    bound = bound + np.ldexp(1.0, np.frexp(np.abs(z))[1] - 9)   # half ulp
                err = np.abs(got - z)
                assert np.all(err <= bound), (seq, lp, h, tensor, float(err.max()))
    # jobs with an out-of-range physical page are skipped: slots 1 and 2 untouched
    assert np.all(kh[1] == 123.0) and np.all(kh[2] == 123.0) and np.all(vh[2] == 123.0)


def test_regen_large_arena_accuracy():
    """16.8 million fp32 values (4 pages of 4096 tokens x 4 heads x 128 dims,
    K and V) against the oracle's fp64 generator: every value within
    1e-6 (1 + |z|).  At this count the Box-Muller inputs reach deep into the
    tails of u (the largest radii), where the hardware log2, square root,
    sine and cosine are least accurate relative to the bound; the worst ratio
    to the bound is printed."""
    import exact_paged_causal_amd as atlas
    hkv, page, d, seed, layer = 4, 4096, 128, 0x5EED5EED, 9
    jobs_np = np.array([[0, 0, 0], [1, 3, 1], [65535, 1, 2], [777, 15, 3]], np.int32)
    say(f"[regen] large arena: {len(jobs_np)} pages x {hkv} heads x {page} x {d}, K and V")
    k = torch.empty((len(jobs_np), hkv, page, d), dtype=torch.float32, device="cuda")
    v = torch.empty_like(k)
    atlas.atlas_regenerate_pages(k, v, torch.from_numpy(jobs_np).cuda(), seed=seed, layer=layer)
    kh, vh = k.cpu().numpy(), v.cpu().numpy()
    worst, n = 0.0, 0
    for seq, lp, phys in jobs_np:
        for h in range(hkv):
            for tensor, arena in ((oracle.TENSOR_K, kh), (oracle.TENSOR_V, vh)):
                z = oracle.regen_rows(seed, layer, int(seq), tensor, h, int(lp) * page, page, d, "f64")
                ratio = np.abs(arena[phys, h].astype(np.float64) - z) / (1e-6 * (1 + np.abs(z)))
                worst = max(worst, float(ratio.max()))
                n += z.size
    say(f"[regen] {n} values, worst ratio to the bound {worst:.3f}")
    assert worst <= 1.0


def test_regen_skips_keys_beyond_16_bits():
    """The generator's counter holds 16 bits of the sequence key: a job with
    seq >= 65536 (or < 0) is skipped, never folded onto seq mod 65536."""
    import exact_paged_causal_amd as atlas
    say("[regen] jobs with sequence keys outside [0, 65536)")
    k = torch.full((3, 1, 8, 64), 123.0, dtype=torch.float32, device="cuda")
    v = torch.full_like(k, 123.0)
    jobs = torch.tensor([[65536, 0, 0], [-1, 0, 1], [3, 0, 2]], dtype=torch.int32, device="cuda")
    atlas.atlas_regenerate_pages(k, v, jobs, seed=1, layer=0)
    torch.cuda.synchronize()
    assert torch.all(k[:2] == 123.0) and torch.all(v[:2] == 123.0)
    assert not torch.any(k[2] == 123.0)


def test_regen_is_placement_free_and_deterministic():
    import exact_paged_causal_amd as atlas
    say("[regen] same logical page into two slots, twice")
    k = torch.zeros((4, 2, 32, 64), dtype=torch.float32, device="cuda")
    v = torch.zeros_like(k)
    jobs = torch.tensor([[3, 9, 0], [3, 9, 2]], dtype=torch.int32, device="cuda")
    atlas.atlas_regenerate_pages(k, v, jobs, seed=5, layer=1)
    k1 = k.clone()
    atlas.atlas_regenerate_pages(k, v, jobs, seed=5, layer=1)
    torch.cuda.synchronize()
    assert torch.equal(k[0], k[2]) and torch.equal(v[0], v[2])
    assert torch.equal(k, k1)


def test_regen_more_jobs_than_one_grid_column():
    """More jobs than the grid's y dimension holds (65535): the jobs past it
    are taken by the grid stride; an invalid job in between is skipped and the
    ones after it still written."""
    import exact_paged_causal_amd as atlas
    n_jobs, seed, layer = 70001, 77, 2
    say(f"[regen] {n_jobs} one-token jobs (grid-strided)")
    k = torch.full((n_jobs, 1, 1, 64), 123.0, dtype=torch.float32, device="cuda")
    v = torch.full_like(k, 123.0)
    j = np.arange(n_jobs, dtype=np.int32)
    jobs_np = np.stack([j % 7, j, j], axis=1).astype(np.int32)
    bad = 65540
    jobs_np[bad, 2] = n_jobs + 5            # out-of-range physical page: skipped
    atlas.atlas_regenerate_pages(k, v, torch.from_numpy(jobs_np).cuda(), seed=seed, layer=layer)
    kh, vh = k.cpu().numpy(), v.cpu().numpy()
    for idx in (0, 1, 65534, 65535, 65536, bad + 1, n_jobs - 1):
        seq, lp, phys = (int(x) for x in jobs_np[idx])
        for tensor, arena in ((oracle.TENSOR_K, kh), (oracle.TENSOR_V, vh)):
            z = oracle.regen_rows(seed, layer, seq, tensor, 0, lp, 1, 64, "f64")
            err = np.abs(arena[phys, 0].astype(np.float64) - z)
            assert np.all(err <= 1e-6 * (1 + np.abs(z))), (idx, tensor, float(err.max()))
    assert np.all(kh[bad] == 123.0) and np.all(vh[bad] == 123.0)


# ------------------------------------------------------ decode, small cases

DECODE_CASES = [
    # (dtype, hq, hkv, d, page, lens, split_tokens)
    ("f32", 1, 1, 64, 16, (1, 2, 15, 16, 17, 100), 0),
    ("f32", 4, 1, 64, 64, (1, 63, 64, 65, 300), 64),           # MQA
    ("f32", 4, 4, 128, 1, (1, 7, 50), 0),                      # MHA, one-token pages
    ("f32", 8, 2, 64, 512, (513, 1000, 1), 128),               # GQA 4
    ("f32", 16, 2, 128, 32, (97, 1024), 96),                   # GQA 8, odd split size
    ("f32", 32, 2, 64, 16, (200,), 0),                         # group of 16 -> several chunks
    ("bf16", 8, 1, 128, 16, (1, 16, 33, 500), 0),
    ("bf16", 4, 2, 64, 64, (5, 64, 129), 64),
    ("bf16", 16, 8, 128, 128, (300, 1), 0),
    ("bf16", 32, 1, 128, 16, (777, 33), 0),                    # group of 32: two 16-row items
    ("bf16", 3, 1, 64, 8, (100, 40), 32),                      # group of 3
    ("bf16", 8, 8, 64, 1, (70, 2), 16),                        # MHA, one-token pages
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"{c[0]}-h{c[1]}x{c[2]}-d{c[3]}-p{c[4]}")
def test_decode_small(case):
    dtype, hq, hkv, d, page, lens, st = case
    w = small(batch=len(lens), hq=hq, hkv=hkv, d=d, page=page, dtype=dtype, lens=lens)
    say(f"[decode-small] {case}")
    inp = H.build(w)
    out, lse = H.run(inp, split_tokens=st)
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what=str(case))


VARIANT_CASES = [
    # (dtype, lens, window, sinks, softcap)
    ("f32", (40, 40, 40, 40), (1, 1, 5, 16), (0, 3, 2, 0), (0.0, 0.0, 0.0, 0.0)),
    ("f32", (64, 65, 300), (0, 0, 0), (0, 0, 0), (1.0, 2.5, 4.0)),
    ("f32", (300, 301), (17, 64), (4, 70), (3.0, 0.0)),
    ("bf16", (100, 1, 33), (7, 1, 40), (4, 1, 0), (2.0, 1.0, 0.0)),
]


@pytest.mark.parametrize("case", VARIANT_CASES, ids=lambda c: f"{c[0]}-w{c[2][0]}")
def test_decode_variants_small(case):
    """Small windows, sinks and caps, where an off-by-one or a wrong softcap
    order moves the output far beyond the tolerance."""
    dtype, lens, win, snk, cap = case
    w = small(batch=len(lens), hq=4, hkv=2, d=64, page=8, dtype=dtype, lens=lens, window=win,
              sinks=snk, softcap=cap)
    say(f"[decode-variants] {case}")
    inp = H.build(w)
    out, lse = H.run(inp, split_tokens=16)
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what=str(case))


MIXED_CASES = [
    # (hq, hkv, d, page, q_len, lens, window, sinks, softcap): fp32 queries over bf16 pages
    (8, 1, 128, 16, 1, (1, 16, 33, 500), None, None, None),
    (4, 2, 64, 64, 1, (5, 64, 129), (0, 20, 0), (0, 2, 0), (0.0, 0.0, 3.0)),
    (32, 1, 128, 16, 1, (777, 33), None, None, None),              # two 16-row items per K/V head
    (8, 2, 128, 16, 9, (9, 300), None, None, None),                # short prefill
    (4, 2, 64, 32, 70, (70, 200), (16, 0), (3, 0), (0.0, 2.0)),    # q_len >= 64 stays on the split path
]


@pytest.mark.parametrize("case", MIXED_CASES, ids=lambda c: f"h{c[0]}x{c[1]}-d{c[2]}-p{c[3]}-q{c[4]}")
def test_f32_query_over_bf16_cache(case):
    """q_dtype f32 with kv_dtype bf16: the bf16 fold carries each query
    element as a bf16 high part and remainder; the bar is the bf16 one (the
    K/V inputs are bf16)."""
    hq, hkv, d, page, q_len, lens, win, snk, cap = case
    w = small(batch=len(lens), hq=hq, hkv=hkv, d=d, page=page, dtype="bf16", q_dtype="f32", q_len=q_len,
              lens=lens, window=win, sinks=snk, softcap=cap)
    say(f"[f32-q/bf16-kv] {case}")
    inp = H.build(w)
    assert inp.q.dtype == torch.float32 and inp.k.dtype == torch.bfloat16
    out, lse = H.run(inp, split_tokens=64)
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what=str(case))


def test_f32_query_mixed_decode_full_size():
    """The mixed-length bf16 decode with fp32 queries, every sequence."""
    w = workloads.make("mixed_decode", q_dtype="f32")
    say("[f32-q/bf16-kv] mixed_decode full size")
    inp = H.build(w)
    out, lse = H.run(inp)
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what="mixed_decode f32 queries")


def test_side_stream_call_matches_current_stream():
    """A call on a caller's side stream (buffers the binding allocates belong
    to that stream) gives the bits of the same call on the current stream."""
    import exact_paged_causal_amd as atlas
    w = small(batch=3, hq=8, hkv=2, d=128, page=16, dtype="bf16", lens=(900, 33, 4000))
    say("[stream] side stream vs current stream")
    inp = H.build(w)
    ref_o, ref_l = H.run(inp)
    ref_o, ref_l = ref_o.clone(), ref_l.clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(4):
        # the binding allocates out, lse and the workspace; garbage on the
        # current stream in between must not disturb the side stream's call
        o, l = atlas.atlas_attend_decode(inp.q, inp.k, inp.v, inp.page_table, inp.context_lens, w.scale,
                                         stream=side)
        junk = torch.full((1 << 20,), 3.0, device="cuda")
        del junk
        outs.append((o, l))
    side.synchronize()
    torch.cuda.synchronize()
    for o, l in outs:
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


def test_custom_head_map():
    hm = [1, 0, 2, 2, 0, 1, 1]
    w = small(batch=2, hq=7, hkv=3, d=64, page=16, lens=(50, 129))
    say("[head-map]", hm)
    inp = H.build(w)
    out, lse = H.run(inp, head_map=hm)
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, head_map=hm, what="head_map")


# ------------------------------------------------- prefill (split-KV path)

PREFILL_CASES = [
    # (dtype, hq, hkv, d, page, q_len, lens, window, sinks, softcap)
    ("f32", 4, 2, 64, 16, 2, (2, 40), None, None, None),
    ("f32", 8, 2, 64, 64, 16, (256,), None, None, None),
    ("f32", 2, 1, 128, 8, 37, (37, 100), None, None, None),
    ("f32", 4, 1, 64, 16, 20, (20, 90), (5, 30), (2, 0), (0.0, 3.0)),
    ("bf16", 8, 2, 128, 16, 9, (9, 300), None, None, None),
    ("bf16", 4, 4, 64, 32, 70, (70, 200), (16, 0), (3, 0), (0.0, 2.0)),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: f"{c[0]}-q{c[5]}-d{c[3]}")
def test_prefill_split_small(case):
    dtype, hq, hkv, d, page, q_len, lens, win, snk, cap = case
    w = small(batch=len(lens), hq=hq, hkv=hkv, d=d, page=page, dtype=dtype, q_len=q_len, lens=lens,
              window=win, sinks=snk, softcap=cap)
    say(f"[prefill-split] {case}")
    inp = H.build(w)
    out, lse = H.run(inp, entry="prefill", split_tokens=32)
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what=str(case))


# --------------------------------------------------- the named workloads

def test_single_head_decode_resident_and_cold():
    """4096-token single-head decode: pages resident (regenerated once) and
    all cold (regenerated on the call) give the same bits, and match."""
    w = workloads.make("single_head_decode")
    say("[single_head_decode] resident")
    inp = H.build(w)
    out, lse = H.run(inp)
    say("[single_head_decode] all cold")
    cold = H.build(workloads.make("single_head_decode", hot_fraction=0.0))
    out_c, lse_c = H.run(cold)
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what="single_head_decode")
    assert torch.equal(out, out_c) and torch.equal(lse, lse_c)


def test_gqa_short_query_in_order_and_shuffled():
    w = workloads.make("gqa_short_query")
    say("[gqa_short_query] in order")
    inp = H.build(w)
    out, lse = H.run(inp)
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what="gqa_short_query")
    say("[gqa_short_query] shuffled pages")
    shuf = H.build(workloads.make("gqa_short_query", shuffle_pages=True))
    out_s, lse_s = H.run(shuf)
    torch.cuda.synchronize()
    assert torch.equal(out, out_s) and torch.equal(lse, lse_s)


def test_long_context_decode_full_size():
    """8 x 65536-token fp32 decode, 25 % resident, the rest regenerated into
    scratch by the call; every (sequence, q-head) checked."""
    w = workloads.make("long_context_decode")
    say("[long_context_decode] full size")
    inp = H.build(w)
    out, lse = H.run(inp)
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what="long_context_decode")


def test_mixed_decode_full_size():
    """64 mixed-length bf16 sequences, window+sinks+softcap on even ones;
    every (sequence, q-head) against the oracle."""
    w = workloads.make("mixed_decode")
    say("[mixed_decode] full size")
    inp = H.build(w)
    out, lse = H.run(inp)
    torch.cuda.synchronize()
    say("[mixed_decode] oracle on all 64 sequences")
    H.check_against_oracle(inp, out, lse, what="mixed_decode")


# ------------------------------------------------------------ invariances

def _reduced_long():
    return workloads.make("long_context_decode", batch=3, context_lens=np.array([8192, 5000, 1], np.int32))


def test_invariant_to_physical_order_and_hot_budget():
    """CFR-Atlas "Core contract": admission changes latency only.  Bit-identical
    outputs across physical placements and resident fractions 0/25/100 %."""
    ref = None
    for hot, seed in [(0.25, 0), (0.0, 1), (1.0, 2), (0.25, 3)]:
        say(f"[invariance] hot={hot} layout_seed={seed}")
        inp = H.build(_reduced_long(), hot_fraction=hot, layout_seed=seed)
        out, lse = H.run(inp)
        torch.cuda.synchronize()
        if ref is None:
            ref = (out.clone(), lse.clone())
            H.check_against_oracle(inp, out, lse, what="invariance reference")
        else:
            assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1])


def test_page_size_changes_only_rounding():
    outs = []
    for page in (16, 64, 512):
        say(f"[page-size] P={page}")
        w = workloads.make("long_context_decode", batch=2, page_size=page,
                           context_lens=np.array([3000, 777], np.int32))
        inp = H.build(w)
        out, lse = H.run(inp, split_tokens=1024)
        torch.cuda.synchronize()
        outs.append((inp, out, lse))
    for inp, out, lse in outs:
        H.check_against_oracle(inp, out, lse, what=f"page size {inp.w.page_size}")
    # same split cuts and key order: the same fold, bit for bit
    assert torch.equal(outs[0][1], outs[1][1]) and torch.equal(outs[0][1], outs[2][1])


def test_nan_poison_outside_the_contexts():
    """Unused arena pages and the tails of last pages hold NaN: outputs are
    bit-identical to the clean run."""
    w = small(batch=3, hq=8, hkv=2, d=128, page=16, dtype="bf16", lens=(17, 100, 33))
    say("[poison] bf16")
    clean = H.build(w)
    o1, l1 = H.run(clean)
    dirty = H.build(w, poison=True, extra_phys=5)
    o2, l2 = H.run(dirty)
    torch.cuda.synchronize()
    assert not torch.isnan(o2).any()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    wr = workloads.make("long_context_decode", batch=2, context_lens=np.array([1500, 700], np.int32))
    say("[poison] regenerated f32")
    a = H.build(wr)
    b = H.build(wr, poison=True, extra_phys=3)
    oa, la = H.run(a)
    ob, lb = H.run(b)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(la, lb)


def test_deterministic_repeat():
    w = workloads.make("long_context_decode", batch=2, context_lens=np.array([20000, 9000], np.int32))
    say("[determinism]")
    inp = H.build(w)
    o1, l1 = H.run(inp)
    o1, l1 = o1.clone(), l1.clone()
    o2, l2 = H.run(inp)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ----------------------------------------------------------- error paths

def test_errors_leave_outputs_untouched():
    import exact_paged_causal_amd as atlas
    w = small(batch=2, hq=4, hkv=2, d=64, page=16, lens=(30, 40))
    say("[errors] small workspace")
    inp = H.build(w)
    out = torch.full((2, 1, 4, 64), 7.0, device="cuda")
    ws = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(atlas.AtlasError) as ei:
        atlas.atlas_attend_decode(inp.q, inp.k, inp.v, inp.page_table, inp.context_lens, w.scale,
                                  out=out, workspace=ws)
    assert ei.value.status == atlas.ATLAS_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_validation_mode_catches_device_side_errors(monkeypatch):
    import exact_paged_causal_amd as atlas
    monkeypatch.setenv("ATLAS_VALIDATE", "1")
    w = small(batch=2, hq=4, hkv=2, d=64, page=16, lens=(30, 40))
    say("[validate] clean call")
    inp = H.build(w)
    out, lse = H.run(inp)
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what="validated call")
    say("[validate] page id outside the pool")
    bad_pt = inp.page_table.clone()
    bad_pt[1, 2] = inp.k.shape[0] + 5
    with pytest.raises(atlas.AtlasError) as ei:
        atlas.atlas_attend_decode(inp.q, inp.k, inp.v, bad_pt, inp.context_lens, w.scale)
    assert ei.value.status == atlas.ATLAS_ERR_POOL
    say("[validate] context longer than the page table")
    bad_ctx = torch.tensor([30, 10**6], dtype=torch.int32, device="cuda")
    with pytest.raises(atlas.AtlasError) as ei:
        atlas.atlas_attend_decode(inp.q, inp.k, inp.v, inp.page_table, bad_ctx, w.scale)
    assert ei.value.status == atlas.ATLAS_ERR_RANGE
    say("[validate] NaN in a visible K row")
    k2 = inp.k.clone()
    k2[int(inp.layout.page_table[0, 1]), 1, 3, 5] = float("nan")
    with pytest.raises(atlas.AtlasError) as ei:
        atlas.atlas_attend_decode(inp.q, k2, inp.v, inp.page_table, inp.context_lens, w.scale)
    assert ei.value.status == atlas.ATLAS_ERR_NONFINITE

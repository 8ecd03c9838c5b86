"""GPU parity of the tiled causal prefill (bf16 matrix-core path) against the
fp64 oracle, through the C ABI.  Each test prints its case before running."""
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
    import exact_paged_causal_amd  # noqa: F401
    yield


def say(*a):
    print(*a, flush=True)


def wl(*, hq, hkv, d, page, q_len, lens, seed=21):
    lens = np.asarray(lens, np.int32)
    return workloads.Workload("prefill_case", seed=seed, batch=len(lens), hq=hq, hkv=hkv, head_dim=d,
                              page_size=page, dtype="bf16", q_len=q_len, context_lens=lens,
                              scale=1.0 / math.sqrt(d), shuffle_pages=True)


CASES = [
    # (hq, hkv, d, page, q_len, lens)
    (4, 1, 128, 16, 64, (64,)),              # one query block, MQA group of 4
    (8, 2, 128, 128, 100, (100, 300)),       # suffix queries; ragged last block
    (2, 2, 64, 32, 257, (257, 400)),         # MHA: 256 positions per block + a 1-row block
    (6, 2, 128, 1, 70, (80,)),               # group of 3 (one padding row), one-token pages
    (16, 1, 64, 64, 96, (200, 96)),          # group of 16
    (32, 8, 128, 128, 512, (512,)),          # the causal-prefill shape, reduced
    (8, 8, 128, 16, 130, (1000,)),           # long history behind a short prefill
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"h{c[0]}x{c[1]}-d{c[2]}-p{c[3]}-q{c[4]}")
def test_tiled_prefill_small(case):
    hq, hkv, d, page, q_len, lens = case
    w = wl(hq=hq, hkv=hkv, d=d, page=page, q_len=q_len, lens=lens)
    say(f"[prefill-tiled] {case}")
    inp = H.build(w)
    out, lse = H.run(inp, entry="prefill")
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what=str(case))


def wlv(*, hq, hkv, d, page, q_len, lens, window, sinks, softcap, seed=23):
    w = wl(hq=hq, hkv=hkv, d=d, page=page, q_len=q_len, lens=lens, seed=seed)
    w.window = np.asarray(window, np.int32)
    w.sinks = np.asarray(sinks, np.int32)
    w.softcap = np.asarray(softcap, np.float32)
    return w


VARIANT_CASES = [
    # (hq, hkv, d, page, q_len, lens, window, sinks, softcap)
    (4, 1, 128, 16, 200, (700, 300), (64, 0), (4, 0), (0.0, 0.0)),         # window + sinks / plain
    (8, 2, 128, 32, 130, (900,), (1,), (0,), (0.0,)),                       # W = 1: own row only
    (8, 2, 128, 32, 130, (900,), (1,), (3,), (2.0,)),                       # W = 1 + 3 sinks + cap 2
    (8, 2, 64, 64, 300, (5000, 300), (100, 4096), (70, 4), (5.0, 0.0)),     # sinks span two blocks; W > ctx
    (2, 2, 128, 128, 257, (3000,), (0,), (0,), (1.5,)),                     # softcap only
    (32, 8, 128, 128, 512, (8192,), (4096,), (4,), (50.0,)),                # the mixed-decode variants on a long prefill
]


@pytest.mark.parametrize("case", VARIANT_CASES, ids=lambda c: f"h{c[0]}x{c[1]}-d{c[2]}-q{c[4]}-w{c[6][0]}")
def test_tiled_prefill_variants(case):
    """Window, sinks and softcap on the tiled path: key blocks before a
    query block's window are skipped, partially visible ones masked."""
    hq, hkv, d, page, q_len, lens, window, sinks, softcap = case
    w = wlv(hq=hq, hkv=hkv, d=d, page=page, q_len=q_len, lens=lens, window=window, sinks=sinks,
            softcap=softcap)
    say(f"[prefill-tiled variants] {case}")
    inp = H.build(w)
    out, lse = H.run(inp, entry="prefill")
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what=str(case))


def test_tiled_prefill_uneven_head_map():
    hm = [0, 1, 1, 0, 1]
    w = wl(hq=5, hkv=2, d=128, page=32, q_len=90, lens=(90, 150))
    say("[prefill-tiled] head map", hm)
    inp = H.build(w)
    out, lse = H.run(inp, entry="prefill", head_map=hm)
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, head_map=hm, what="uneven head map")


def test_causal_prefill_full_size():
    """S=8192, Hq=32, Hkv=8, D=128, pages of 128 in random physical order:
    every row of one seeded q-head per K/V head, and the first and last 512
    rows of every q-head, against the oracle; no NaN anywhere."""
    w = workloads.make("causal_prefill")
    say("[causal_prefill] full size")
    inp = H.build(w)
    out, lse = H.run(inp)
    torch.cuda.synchronize()
    for rows, heads in H.full_size_blocks(w, seed=0):
        say(f"[causal_prefill] oracle on {len(rows)} rows x heads {heads.tolist()}")
        H.check_against_oracle(inp, out, lse, rows=rows, heads=heads, what="causal_prefill")
    assert not torch.isnan(out).any() and not torch.isnan(lse).any()


def restage_workload(dtype, hkv=8, ctx=33000, q_len=64, window=None, sinks=None, softcap=None, seed=25):
    """32 sequences x hkv K/V heads, pages of 16, q_len positions each: 256
    workgroups fill the chip, so no key splits; each workgroup's key range
    spans more pages than its page-id window holds (2048 pages for bf16,
    1024 for fp32), so the window is restaged inside the key loop."""
    B = 256 // hkv
    lens = np.full(B, ctx, np.int32)
    lens[1::2] -= 333                       # ragged last pages
    w = workloads.Workload("restage", seed=seed, batch=B, hq=hkv, hkv=hkv, head_dim=128, page_size=16,
                           dtype=dtype, q_len=q_len, context_lens=lens, scale=1.0 / math.sqrt(128),
                           shuffle_pages=True)
    if window is not None:
        w.window, w.sinks, w.softcap = (np.asarray(x, np.int32 if i < 2 else np.float32)
                                        for i, x in enumerate((window, sinks, softcap)))
    return w


def test_tiled_prefill_restages_page_ids():
    """bf16 tiled prefill whose workgroups each read 33000 keys in pages of
    16 (2063 pages, above the 2048-entry page-id window), and windowed rows
    (window 100 + 4 sinks) whose first window block sits more than 2048
    pages after the sink page: both restage the window.  Two sequences of
    each kind against the oracle."""
    B = 32
    win = np.where(np.arange(B) % 4 == 0, 100, 0)
    snk = np.where(np.arange(B) % 4 == 0, 4, 0)
    cap = np.zeros(B, np.float32)
    w = restage_workload("bf16", window=win, sinks=snk, softcap=cap)
    say("[prefill-tiled] page-id window restage (33000 keys in pages of 16)")
    inp = H.build(w)
    out, lse = H.run(inp, entry="prefill")
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, seqs=[0, 4, 1, 3], what="restage")
    assert not torch.isnan(out).any()


def test_tiled_prefill_poison_and_determinism():
    w = wl(hq=8, hkv=2, d=128, page=16, q_len=100, lens=(117, 100, 300))
    say("[prefill-tiled] poison")
    clean = H.build(w)
    o1, l1 = H.run(clean, entry="prefill")
    o1, l1 = o1.clone(), l1.clone()
    dirty = H.build(w, poison=True, extra_phys=4)
    o2, l2 = H.run(dirty, entry="prefill")
    o3, l3 = H.run(dirty, entry="prefill")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o2, o3) and torch.equal(l2, l3)
    H.check_against_oracle(clean, o1, l1, what="poison reference")


def test_tiled_prefill_invariant_to_page_order():
    base = wl(hq=8, hkv=2, d=64, page=16, q_len=200, lens=(200, 333))
    say("[prefill-tiled] page order")
    a = H.build(base, layout_seed=0)
    b = H.build(base, layout_seed=5)
    oa, la = H.run(a, entry="prefill")
    ob, lb = H.run(b, entry="prefill")
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(la, lb)


def test_validation_rejects_v_beyond_fp16(monkeypatch):
    import exact_paged_causal_amd as atlas
    monkeypatch.setenv("ATLAS_VALIDATE", "1")
    w = wl(hq=4, hkv=1, d=128, page=16, q_len=64, lens=(64,))
    say("[prefill-tiled] validation of the fp16 range")
    inp = H.build(w)
    v2 = inp.v.clone()
    v2[int(inp.layout.page_table[0, 0]), 0, 2, 7] = 1.0e5
    with pytest.raises(atlas.AtlasError) as ei:
        atlas.atlas_attend_prefill(inp.q, inp.k, v2, inp.page_table, inp.context_lens, w.scale)
    assert ei.value.status == atlas.ATLAS_ERR_RANGE
    out, lse = H.run(inp, entry="prefill")   # the clean input passes validation
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what="validated prefill")

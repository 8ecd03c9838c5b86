"""GPU parity of the fp32 tiled prefill (fp16 matrix cores with split
operands) against the fp64 oracle, through the C ABI, at the fp32 bar
(|gpu - ref| <= 2e-5 + 1e-4 |ref|).  Each test prints its case before
running."""
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


def wl(*, hq, hkv, d, page, q_len, lens, seed=31, window=None, sinks=None, softcap=None):
    lens = np.asarray(lens, np.int32)
    w = workloads.Workload("prefill_f32_case", seed=seed, batch=len(lens), hq=hq, hkv=hkv, head_dim=d,
                           page_size=page, dtype="f32", q_len=q_len, context_lens=lens,
                           scale=1.0 / math.sqrt(d), shuffle_pages=True)
    if window is not None:
        w.window = np.asarray(window, np.int32)
        w.sinks = np.asarray(sinks, np.int32)
        w.softcap = np.asarray(softcap, np.float32)
    return w


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
def test_f32_tiled_prefill_small(case):
    hq, hkv, d, page, q_len, lens = case
    say(f"[prefill-f32] {case}")
    inp = H.build(wl(hq=hq, hkv=hkv, d=d, page=page, q_len=q_len, lens=lens))
    out, lse = H.run(inp, entry="prefill")
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what=str(case))


VARIANT_CASES = [
    # (hq, hkv, d, page, q_len, lens, window, sinks, softcap)
    (4, 1, 128, 16, 200, (700, 300), (64, 0), (4, 0), (0.0, 0.0)),         # window + sinks / plain
    (8, 2, 128, 32, 130, (900,), (1,), (3,), (2.0,)),                       # W = 1 + 3 sinks + cap 2
    (8, 2, 64, 64, 300, (5000, 300), (100, 4096), (70, 4), (5.0, 0.0)),     # sinks span two blocks; W > ctx
    (2, 2, 128, 128, 257, (3000,), (0,), (0,), (30.0,)),                    # softcap only
]


@pytest.mark.parametrize("case", VARIANT_CASES, ids=lambda c: f"h{c[0]}x{c[1]}-d{c[2]}-q{c[4]}-w{c[6][0]}")
def test_f32_tiled_prefill_variants(case):
    hq, hkv, d, page, q_len, lens, window, sinks, softcap = case
    say(f"[prefill-f32] variants {case}")
    inp = H.build(wl(hq=hq, hkv=hkv, d=d, page=page, q_len=q_len, lens=lens, window=window, sinks=sinks,
                     softcap=softcap))
    out, lse = H.run(inp, entry="prefill")
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what=f"variants {case}")


@pytest.mark.parametrize("qs,ks,vs,at_data_scale", [
    (2.0 ** -10, 2.0 ** 10, 1.0, False),   # Q lo parts in the fp16 subnormal range
    (4.0, 0.25, 2.0 ** 10, True),          # large V: hi parts near 2^12
    (1.0, 1.0, 2.0 ** -10, False),         # small V: lo parts subnormal, absolute bar
], ids=["tiny-q", "large-v", "tiny-v"])
def test_f32_tiled_prefill_magnitudes(qs, ks, vs, at_data_scale):
    """Inputs scaled by powers of two (exact) so that the split parts cover
    the fp16 range (subnormal lo parts, large hi parts) while the logits stay
    of order one.  The bar's absolute term is in units of the data: with V
    scaled up by 2^10 the output, which averages values of that size, is
    compared after dividing by the scale (against the oracle on the unscaled
    V), as fp32 arithmetic itself rounds at that scale."""
    w = wl(hq=8, hkv=2, d=128, page=16, q_len=150, lens=(150, 400))
    say(f"[prefill-f32] magnitudes q*{qs} k*{ks} v*{vs}")
    inp = H.build(w)
    inp.q.mul_(qs)
    inp.k.mul_(ks)
    inp.v.mul_(vs)
    out, lse = H.run(inp, entry="prefill")
    torch.cuda.synchronize()
    if at_data_scale:
        inp.v.div_(vs)
        out = out / vs
    H.check_against_oracle(inp, out, lse, what=f"magnitudes {qs} {ks} {vs}")


def test_f32_tiled_prefill_uneven_head_map():
    hm = [0, 1, 1, 0, 1]
    w = wl(hq=5, hkv=2, d=64, page=32, q_len=90, lens=(90, 150))
    say("[prefill-f32] head map", hm)
    inp = H.build(w)
    out, lse = H.run(inp, entry="prefill", head_map=hm)
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, head_map=hm, what="uneven head map")


def test_f32_tiled_prefill_poison_determinism_and_page_order():
    w = wl(hq=8, hkv=2, d=128, page=16, q_len=100, lens=(117, 100, 300))
    say("[prefill-f32] poison, determinism, page order")
    clean = H.build(w)
    o1, l1 = H.run(clean, entry="prefill")
    o1, l1 = o1.clone(), l1.clone()
    dirty = H.build(w, poison=True, extra_phys=4, layout_seed=3)
    o2, l2 = H.run(dirty, entry="prefill")
    o2, l2 = o2.clone(), l2.clone()
    o3, l3 = H.run(dirty, entry="prefill")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o2, o3) and torch.equal(l2, l3)
    H.check_against_oracle(clean, o1, l1, what="poison reference")


def test_f32_causal_prefill_full_size():
    """The causal-prefill shape in fp32 (S=8192, Hq=32, Hkv=8, D=128, pages
    of 128 in random physical order): every row of one seeded q-head per K/V
    head, and the first and last 512 rows of every q-head."""
    w = workloads.make("causal_prefill", dtype="f32")
    say("[prefill-f32] causal_prefill shape, fp32")
    inp = H.build(w)
    out, lse = H.run(inp)
    torch.cuda.synchronize()
    for rows, heads in H.full_size_blocks(w, seed=1):
        say(f"[prefill-f32] oracle on {len(rows)} rows x heads {heads.tolist()}")
        H.check_against_oracle(inp, out, lse, rows=rows, heads=heads, what="causal_prefill f32")
    assert not torch.isnan(out).any() and not torch.isnan(lse).any()


def test_f32_tiled_prefill_restages_page_ids():
    """fp32 tiled prefill over 17000 keys in pages of 16 per workgroup (1063
    pages, above its 1024-entry page-id window), unsplit (256 workgroups),
    with windowed rows whose window starts past page 1024 of their sinks."""
    B = 32
    lens = np.full(B, 17000, np.int32)
    lens[1::2] -= 333
    w = workloads.Workload("restage_f32", seed=35, batch=B, hq=8, hkv=8, head_dim=128, page_size=16,
                           dtype="f32", q_len=64, context_lens=lens, scale=1.0 / math.sqrt(128),
                           shuffle_pages=True)
    w.window = np.where(np.arange(B) % 4 == 0, 300, 0).astype(np.int32)
    w.sinks = np.where(np.arange(B) % 4 == 0, 4, 0).astype(np.int32)
    w.softcap = np.zeros(B, np.float32)
    say("[prefill-f32] page-id window restage (17000 keys in pages of 16)")
    inp = H.build(w)
    out, lse = H.run(inp, entry="prefill")
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, seqs=[0, 4, 1, 3], what="restage f32")
    assert not torch.isnan(out).any()


@pytest.mark.parametrize("qexp,kexp", [(20, -20), (-20, 20), (30, -30), (0, -60)])
def test_f32_tiled_prefill_takes_q_and_k_beyond_fp16(monkeypatch, qexp, kexp):
    """Q and K rows are range-scaled by powers of two inside the kernel, so
    elements far outside the fp16 range (|q| up to ~2^32, |k| down to
    2^-60) are accepted (validation mode too) and meet the fp32 bar.  The
    pairs keep the scores q.k in their usual range (or shrink them): scores
    themselves far beyond it (~1e12) are beyond any fp32 softmax."""
    monkeypatch.setenv("ATLAS_VALIDATE", "1")
    w = wl(hq=8, hkv=2, d=128, page=16, q_len=100, lens=(100, 250))
    say(f"[prefill-f32] q x 2^{qexp}, k x 2^{kexp}")
    inp = H.build(w)
    inp.q.mul_(2.0 ** qexp)
    inp.k.mul_(2.0 ** kexp)
    out, lse = H.run(inp, entry="prefill")
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what=f"q x 2^{qexp}, k x 2^{kexp}")


def test_f32_validation_rejects_v_beyond_fp16(monkeypatch):
    import exact_paged_causal_amd as atlas
    monkeypatch.setenv("ATLAS_VALIDATE", "1")
    w = wl(hq=4, hkv=1, d=64, page=16, q_len=64, lens=(64,))
    say("[prefill-f32] validation of V's fp16 range")
    inp = H.build(w)
    v = inp.v.clone()
    pid = int(inp.layout.page_table[0, 0])
    v[pid, 0, 2, 7] = 1.0e5
    with pytest.raises(atlas.AtlasError) as ei:
        atlas.atlas_attend_prefill(inp.q, inp.k, v, inp.page_table, inp.context_lens, w.scale)
    assert ei.value.status == atlas.ATLAS_ERR_RANGE
    out, lse = H.run(inp, entry="prefill")   # the clean input passes validation
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what="validated fp32 prefill")
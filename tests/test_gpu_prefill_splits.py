"""GPU parity of the tiled prefills with key splits (short prefill chunks
behind long histories, where the query blocks alone would leave most CUs
idle): each workgroup folds a run of its query block's key blocks and the
LSE merge combines the runs.  Against the fp64 oracle, bf16 and fp32, with
windows / sinks / softcap and with atlas_attend_mods.  Each test prints its
case before running."""
import math

import numpy as np
import pytest
import torch

import harness as H
import workloads
from test_gpu_mods import alibi_slopes, check_mods, make_mask, run_mods

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_paged_causal_amd  # noqa: F401  (fails loudly if libatlas.so is missing)
    yield


def say(*a):
    print(*a, flush=True)


def wl(dtype, hq, hkv, d, page, q_len, lens, seed=51, window=None, sinks=None, softcap=None):
    lens = np.asarray(lens, np.int32)
    w = workloads.Workload("split_case", seed=seed, batch=len(lens), hq=hq, hkv=hkv, head_dim=d, page_size=page,
                           dtype=dtype, q_len=q_len, context_lens=lens, scale=1.0 / math.sqrt(d), shuffle_pages=True)
    if window is not None:
        w.window = np.asarray(window, np.int32)
        w.sinks = np.asarray(sinks, np.int32)
        w.softcap = np.asarray(softcap, np.float32)
    return w


def split_count(inp, head_map=None):
    """Workspace beyond the 256-byte header: the partial states of the splits."""
    import exact_paged_causal_amd as atlas
    args, _ = atlas.make_attn_args(inp.q, inp.k, inp.v, inp.page_table, inp.context_lens, inp.w.scale,
                                   head_map=head_map)
    return atlas.atlas_prefill_workspace_bytes(args) - 256


CASES = [
    # (dtype, hq, hkv, d, page, q_len, lens, window, sinks, softcap)
    ("bf16", 32, 8, 128, 64, 128, (20000,), None, None, None),
    ("bf16", 8, 2, 128, 16, 200, (9000, 3000), (1000, 0), (4, 0), (30.0, 0.0)),
    ("bf16", 16, 1, 64, 128, 64, (30000,), None, None, None),
    ("f32", 32, 8, 128, 64, 128, (12000,), None, None, None),
    ("f32", 8, 2, 64, 32, 300, (7000, 400), (2000, 0), (0, 0), (0.0, 10.0)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-h{c[1]}x{c[2]}-d{c[3]}-q{c[5]}-L{c[6][0]}"
                                                     f"{'-win' if c[7] else ''}")
def test_key_splits_match_oracle(case):
    dtype, hq, hkv, d, page, q_len, lens, win, snk, cap = case
    say(f"[splits] {case}")
    inp = H.build(wl(dtype, hq, hkv, d, page, q_len, lens, window=win, sinks=snk, softcap=cap), poison=True)
    assert split_count(inp) > 0, "this shape should take key splits"
    out, lse = H.run(inp, entry="prefill")
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what=str(case))


@pytest.mark.parametrize("dtype,causal,alibi,density", [
    ("bf16", False, True, 0.6), ("bf16", True, True, None), ("f32", False, False, 0.5), ("f32", True, True, 0.8),
])
def test_key_splits_with_mods(dtype, causal, alibi, density):
    w = wl(dtype, 8, 2, 128, 32, 100, (8000, 5000))
    say(f"[splits] mods {dtype} causal={causal} alibi={alibi} mask={density}")
    inp = H.build(w, poison=True)
    assert split_count(inp) > 0
    slopes = alibi_slopes(8) if alibi else None
    mask = make_mask(w, density, seed=12) if density else None
    out, lse = run_mods(inp, causal, slopes, mask)
    torch.cuda.synchronize()
    check_mods(inp, out, lse, causal, slopes, mask, f"splits mods {dtype}")


def test_key_splits_are_deterministic():
    w = wl("bf16", 32, 8, 128, 64, 128, (20000,))
    say("[splits] determinism")
    inp = H.build(w)
    o1, l1 = H.run(inp, entry="prefill")
    o1, l1 = o1.clone(), l1.clone()
    o2, l2 = H.run(inp, entry="prefill")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_key_splits_one_token_pages_and_uneven_head_map(dtype):
    """Key splits over one-token pages, with an uneven q-head -> K/V-head map
    (groups of 3 and 2: padded rows in every query block)."""
    hm = [0, 1, 1, 0, 1]
    w = wl(dtype, 5, 2, 64, 1, 96, (3000, 1200))
    say(f"[splits] one-token pages, head map {hm}, {dtype}")
    inp = H.build(w)
    assert split_count(inp, hm) > 0
    out, lse = H.run(inp, entry="prefill", head_map=hm)
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, head_map=hm, what=f"one-token pages {dtype}")


def test_key_splits_with_a_long_page_table():
    """max_pages_per_seq far beyond the contexts: the split count comes from
    the largest possible context, most runs find no block and return."""
    w = wl("bf16", 8, 2, 128, 16, 80, (2000, 100))
    say("[splits] long page table")
    inp = H.build(w, extra_phys=8)
    pt = torch.full((w.batch, 4096), 0, dtype=torch.int32, device="cuda")
    pt[:, :inp.page_table.shape[1]] = inp.page_table
    import exact_paged_causal_amd as atlas
    out, lse = atlas.atlas_attend_prefill(inp.q, inp.k, inp.v, pt, inp.context_lens, w.scale)
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what="long page table")

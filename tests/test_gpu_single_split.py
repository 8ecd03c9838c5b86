"""GPU parity of calls whose plan gives every row a single split (contexts up
to 256 keys without a sink array): the fold writes each row's final output
and lse itself and no merge is launched.  Checked against the fp64 oracle
across dtype pairs, head dims, query counts, windows, softcaps, the
modifications and in-kernel regeneration; and on device lengths shorter than
the query count (rows that see no key come back NaN with lse = -inf, the
others match the oracle), on this path and on the merge path.  Each test
prints its case first."""
import dataclasses
import math
import os

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


def wl(dtype, hq, hkv, d, page, q_len, lens, q_dtype=None, window=None, softcap=None, seed=61, **kw):
    w = workloads.Workload("single_split", seed=seed, batch=len(lens), hq=hq, hkv=hkv, head_dim=d, page_size=page,
                           dtype=dtype, q_len=q_len, context_lens=np.asarray(lens, np.int32),
                           scale=1.0 / math.sqrt(d), shuffle_pages=True, q_dtype=q_dtype, **kw)
    if window is not None:
        w.window = np.asarray(window, np.int32)
        w.softcap = np.asarray(softcap, np.float32)
    return w


def one_split(w, entry, max_pages):
    """The plan's workspace holds one partial state per row: a single split."""
    from exact_paged_causal_amd import atlas as A
    a = A.AttnArgs()
    a.q_dtype = 0 if (w.q_dtype or w.dtype) == "f32" else 1
    a.kv_dtype = 0 if w.dtype == "f32" else 1
    a.batch, a.q_len, a.num_q_heads, a.num_kv_heads, a.head_dim = w.batch, w.q_len, w.hq, w.hkv, w.head_dim
    a.page_size, a.num_phys_pages = w.page_size, 1 << 20
    a.max_pages_per_seq = int(max_pages)
    a.scale = w.scale
    fn = A.atlas_decode_workspace_bytes if entry == "decode" else A.atlas_prefill_workspace_bytes
    rows = w.batch * w.q_len * w.hq
    return fn(a) == 256 + rows * (w.head_dim + 2) * 4


CASES = [
    # (dtype, q_dtype, hq, hkv, d, page, q_len, lens, window / softcap)
    ("f32", None, 8, 2, 64, 64, 16, (256,), None),          # the GQA short query's shape
    ("f32", None, 4, 1, 64, 16, 1, (256, 37, 1), None),
    ("f32", None, 8, 8, 128, 1, 7, (200, 9), ((16, 0), (0.0, 30.0))),
    ("bf16", None, 32, 8, 128, 16, 1, (256, 100, 17, 250), None),
    ("bf16", None, 16, 2, 64, 2, 33, (256, 40), ((20, 5), (2.0, 0.0))),
    ("bf16", "f32", 8, 1, 128, 64, 1, (256, 129), None),
    ("bf16", "f32", 4, 2, 64, 16, 12, (90, 256), ((0, 8), (0.0, 5.0))),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}{'-q' + c[1] if c[1] else ''}-h{c[2]}x{c[3]}-d{c[4]}"
                                                     f"-p{c[5]}-q{c[6]}-L{max(c[7])}{'-var' if c[8] else ''}")
def test_single_split_matches_oracle(case):
    dtype, qd, hq, hkv, d, page, q_len, lens, var = case
    say(f"[single-split] {case}")
    w = wl(dtype, hq, hkv, d, page, q_len, lens, q_dtype=qd,
           window=None if var is None else var[0], softcap=None if var is None else var[1])
    entry = "decode" if q_len == 1 else "prefill"
    inp = H.build(w, poison=True, extra_phys=2)
    assert one_split(w, entry, inp.page_table.shape[1])
    out, lse = H.run(inp, entry=entry)
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what=str(case))


@pytest.mark.parametrize("dtype,q_len", [("f32", 1), ("bf16", 9)])
def test_single_split_mods(dtype, q_len):
    """Non-causal rows with ALiBi and a mask (some rows see nothing) on a
    single split."""
    say(f"[single-split] mods {dtype} q_len={q_len}")
    w = wl(dtype, 8, 2, 64, 16, q_len, (256, 64))
    inp = H.build(w, poison=True)
    slopes = alibi_slopes(8)
    mask = make_mask(w, 0.6, seed=12, empty_rows=1)
    out, lse = run_mods(inp, False, slopes, mask)
    torch.cuda.synchronize()
    check_mods(inp, out, lse, False, slopes, mask, f"single split mods {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_split_fused_regeneration(dtype):
    """Cold pages generated in the fold, on a single split, against the
    oracle's own generator."""
    import exact_paged_causal_amd as atlas
    say(f"[single-split] fused regeneration {dtype}")
    w = wl(dtype, 8, 2, 64, 16, 1, (256, 200, 31), regenerated=True, hot_fraction=0.4)
    inp = H.build(w)
    pt = inp.layout.page_table.copy()
    for seq, lp, _ in inp.layout.cold_jobs:
        pt[seq, lp] = atlas.ATLAS_PAGE_REGENERATE
    out, lse = atlas.atlas_attend_decode_regen(inp.q, inp.k, inp.v, torch.from_numpy(pt).cuda(), inp.context_lens,
                                               w.scale, seed=w.seed, layer=w.layer)
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what=f"single split fused {dtype}")


@pytest.mark.parametrize("dtype,lens", [("f32", (200, 256)), ("bf16", (200, 256)), ("f32", (900, 1000)),
                                        ("bf16", (900, 1000))])
def test_rows_without_keys_on_short_lengths(dtype, lens):
    """Device lengths shorter than the query count.  Without validation mode
    (which rejects them with ATLAS_ERR_RANGE), sequence 0's first rows sit
    before position 0 and see nothing (NaN, lse = -inf); its other rows and
    sequence 1 match the oracle over the keys the lengths give.  Lengths up
    to 256 take the single-split path, longer ones the merge."""
    say(f"[single-split] rows without keys, {dtype} lens={lens}")
    q_len = 40
    w = wl(dtype, 8, 2, 64, 16, q_len, lens)
    inp = H.build(w, poison=False)
    short = np.array([25, lens[1]], np.int32)       # 25 < q_len: rows 0..14 see nothing
    ctx = torch.from_numpy(short).cuda()
    import exact_paged_causal_amd as atlas
    if os.environ.get("ATLAS_VALIDATE", "") not in ("", "0"):
        # validation mode reports such lengths instead of running the call
        with pytest.raises(atlas.AtlasError) as ei:
            atlas.atlas_attend_prefill(inp.q, inp.k, inp.v, inp.page_table, ctx, w.scale)
        assert ei.value.status == atlas.ATLAS_ERR_RANGE
        return
    out, lse = atlas.atlas_attend_prefill(inp.q, inp.k, inp.v, inp.page_table, ctx, w.scale)
    torch.cuda.synchronize()
    dead = q_len - 25
    assert torch.isnan(out[0, :dead]).all() and torch.isneginf(lse[0, :dead]).all()
    assert not torch.isnan(out[0, dead:]).any() and not torch.isnan(out[1]).any()
    w2 = dataclasses.replace(w, context_lens=short)
    inp2 = dataclasses.replace(inp, w=w2, context_lens=ctx)
    ref_o, ref_l = H.oracle_answer(inp2, 0, rows=np.arange(dead, q_len))
    H.assert_close(H.to_f32_numpy(out[0, dead:]), ref_o, dtype, "live rows of sequence 0")
    H.assert_close(H.to_f32_numpy(lse[0, dead:]), ref_l, dtype, "live rows of sequence 0 (lse)")
    H.check_against_oracle(inp2, out, lse, seqs=[1], what="sequence 1")

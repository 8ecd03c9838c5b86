"""GPU parity of calls whose rows have more than 64 splits.  A decode of one
or a few sequences over few K/V heads has few (sequence, K/V head, row
chunk) work items per split, so the split plan gives such a call up to 512
splits per row (enough for two work items per CU), and rows with more than
64 splits are merged by eight waves each.  Cases: fp32 and bf16 caches, an
fp32 query over a bf16 cache, contexts of 70000 to 160000 keys, ragged
lengths (rows with 1 to 79 splits in one call), window / sink / softcap
variants, the fused-regeneration decode (bit-identical to regenerating into
scratch first) and a row that sees no key.  Each case asserts the plan's
split count (the ATLAS_DEBUG line) and checks every row against the
oracle."""
import dataclasses
import math
import os
import re

import numpy as np
import pytest
import torch

import harness as H
import workloads
from test_gpu_fused_regen import regen_workload, run_fused

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_paged_causal_amd  # noqa: F401  (fails loudly if libatlas.so is missing)
    yield


def say(*a):
    print(*a, flush=True)


def planned_splits(err):
    m = re.search(r"max_splits=(\d+)", err)
    assert m, f"no plan line in stderr: {err!r}"
    return int(m.group(1))


# (id, kv dtype, q dtype, head_dim, page, hq, hkv, lens, variants, expected max_splits)
CASES = [
    ("f32-h8x1-131072", "f32", None, 128, 128, 8, 1, (131072,), {}, 512),
    ("bf16-h1x1-131072", "bf16", None, 64, 256, 1, 1, (131072,), {}, 512),
    ("bf16-h64x1-100000", "bf16", None, 128, 64, 64, 1, (100000,), {}, 98),
    ("f32q-bf16-h8x1-70000", "bf16", "f32", 128, 16, 8, 1, (70000,), {}, 274),
    ("bf16-h16x2-ragged", "bf16", None, 128, 128, 16, 2, (160000, 5000, 1), {}, 79),
    ("f32-h4x1-variants", "f32", None, 64, 64, 4, 1, (100000, 70000),
     dict(window=(0, 20000), sinks=(0, 5), softcap=(0.0, 30.0)), None),
]


@pytest.mark.parametrize("c", CASES, ids=[c[0] for c in CASES])
def test_many_splits_match_oracle(c, capfd, monkeypatch):
    name, dt, qdt, d, page, hq, hkv, lens, ex, want = c
    say(f"[many-splits] {name} lens={lens}")
    w = workloads.Workload(f"many_{name}", seed=40 + CASES.index(c), batch=len(lens), hq=hq, hkv=hkv, head_dim=d,
                           page_size=page, dtype=dt, q_dtype=qdt, q_len=1, context_lens=np.asarray(lens, np.int32),
                           scale=1.0 / math.sqrt(d), shuffle_pages=True)
    if ex:
        w.window = np.asarray(ex["window"], np.int32)
        w.sinks = np.asarray(ex["sinks"], np.int32)
        w.softcap = np.asarray(ex["softcap"], np.float32)
    inp = H.build(w, poison=True)
    capfd.readouterr()
    monkeypatch.setenv("ATLAS_DEBUG", "1")
    out, lse = H.run(inp, entry="decode")
    torch.cuda.synchronize()
    monkeypatch.delenv("ATLAS_DEBUG")
    err = capfd.readouterr().err
    say(err.strip())
    n = planned_splits(err)
    assert n > 64 and (want is None or n == want), f"{name}: planned {n} splits per row, expected {want}"
    H.check_against_oracle(inp, out, lse, what=name)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_many_splits_fused_regeneration(dtype, capfd, monkeypatch):
    """The fused-regeneration decode of one sequence over 65536 keys (a
    quarter of its pages resident): more than 64 splits per row, the oracle
    over the generator's values, and the same bits as regenerating the cold
    pages into scratch and decoding."""
    w = regen_workload(1, (65536,), d=128, page=256, hq=8, hkv=1, hot=0.25, dtype=dtype)
    say(f"[many-splits] fused regeneration {dtype}")
    inp = H.build(w, poison=True)
    capfd.readouterr()
    monkeypatch.setenv("ATLAS_DEBUG", "1")
    out_f, lse_f = run_fused(inp)
    torch.cuda.synchronize()
    monkeypatch.delenv("ATLAS_DEBUG")
    err = capfd.readouterr().err
    say(err.strip())
    assert planned_splits(err) > 64
    H.check_against_oracle(inp, out_f, lse_f, what=f"fused {dtype}")
    out_s, lse_s = H.run(inp)
    torch.cuda.synchronize()
    assert torch.equal(out_f, out_s) and torch.equal(lse_f, lse_s)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_many_splits_row_without_keys(dtype):
    """A call planned with more than 64 splits per row in which one sequence's
    device length is 0: that row sees no key (NaN, lse = -inf; validation
    mode rejects the length with ATLAS_ERR_RANGE instead), the other matches
    the oracle."""
    import exact_paged_causal_amd as atlas
    w = workloads.Workload("many_dead", seed=47, batch=2, hq=8, hkv=1, head_dim=64, page_size=128, dtype=dtype,
                           q_len=1, context_lens=np.asarray((131072, 5), np.int32), scale=0.125, shuffle_pages=True)
    say(f"[many-splits] row without keys {dtype}")
    inp = H.build(w, poison=False)
    short = np.array([131072, 0], np.int32)
    ctx = torch.from_numpy(short).cuda()
    if os.environ.get("ATLAS_VALIDATE", "") not in ("", "0"):
        with pytest.raises(atlas.AtlasError) as ei:
            atlas.atlas_attend_decode(inp.q, inp.k, inp.v, inp.page_table, ctx, w.scale)
        assert ei.value.status == atlas.ATLAS_ERR_RANGE
        return
    out, lse = atlas.atlas_attend_decode(inp.q, inp.k, inp.v, inp.page_table, ctx, w.scale)
    torch.cuda.synchronize()
    assert torch.isnan(out[1]).all() and torch.isneginf(lse[1]).all()
    w2 = dataclasses.replace(w, context_lens=short)
    inp2 = dataclasses.replace(inp, w=w2, context_lens=ctx)
    H.check_against_oracle(inp2, out, lse, seqs=[0], what="sequence 0")

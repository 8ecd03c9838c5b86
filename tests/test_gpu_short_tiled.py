"""GPU parity of short query blocks (1 to 63 queries per sequence) on both
sides of the tiled-kernel routing bound.  A prefill of fewer than 64 queries
runs the tiled kernels when the split-KV kernels would need several row
chunks per K/V head (queries x group above 32 rows for a bf16 cache, above 8
for fp32) and the call covers at least 2^17 query-key pairs (2^16 for fp32
with two or more queries); otherwise it runs the split-KV kernels.  The
decode entry always runs the split-KV kernels, also where a single query
through the prefill entry is tiled.  Each case asserts which
kernels ran (the ATLAS_DEBUG line) and checks every query row and q-head of
every sequence against the oracle, with plain calls, per-sequence window /
sink / softcap variants, modifications (non-causal rows, ALiBi slopes,
mask bits), 256 q-heads over one K/V head (one query position per
workgroup, with key splits: 65 to 115 partial states per row, so the merge
goes past its first 64) and an uneven head map (the largest group sets the
rows).  NaN-poisoned arenas, shuffled pages; each case prints itself
first."""
import math

import numpy as np
import pytest
import torch

import harness as H
import workloads
from test_gpu_mods import alibi_slopes, check_mods, run_mods

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_paged_causal_amd  # noqa: F401  (fails loudly if libatlas.so is missing)
    yield


# (id, dtype, head_dim, page, hq, hkv, q_len, lens, expected route, extras)
CASES = [
    ("bf16-g4-q9", "bf16", 128, 64, 16, 4, 9, (16384,), "tiled", {}),
    ("bf16-g4-q8", "bf16", 128, 16, 16, 4, 8, (16384, 9000), "split", {}),
    ("bf16-g8-q5", "bf16", 64, 256, 16, 2, 5, (16384, 12000), "tiled", {}),
    ("bf16-g8-q4", "bf16", 64, 64, 16, 2, 4, (16384, 16384), "split", {}),
    ("bf16-g1-q40", "bf16", 128, 1, 4, 4, 40, (4096,), "tiled", {}),
    ("bf16-g1-q32", "bf16", 64, 16, 4, 4, 32, (8192,), "split", {}),
    ("bf16-g4-q16-ragged", "bf16", 64, 16, 8, 2, 16, (16, 9000, 20000), "tiled", {}),
    ("bf16-g4-q9-small", "bf16", 128, 64, 16, 4, 9, (8192,), "split", {}),
    ("f32-g4-q3", "f32", 64, 64, 8, 2, 3, (32768,), "tiled", {}),
    ("f32-g2-q5", "f32", 128, 16, 8, 4, 5, (16384,), "tiled", {}),
    ("f32-g8-q2", "f32", 64, 64, 16, 2, 2, (16384, 16384), "tiled", {}),
    ("f32-g1-q9", "f32", 128, 256, 4, 4, 9, (8192,), "tiled", {}),
    ("f32-g1-q8", "f32", 64, 16, 4, 4, 8, (8192, 8000), "split", {}),
    ("f32-g4-q2", "f32", 64, 64, 8, 2, 2, (2, 30000), "split", {}),
    ("bf16-g4-q12-var", "bf16", 128, 64, 8, 2, 12, (10000, 12000), "tiled",
     dict(window=(0, 700), sinks=(4, 0), softcap=(50.0, 0.0))),
    ("f32-g8-q3-var", "f32", 64, 16, 16, 2, 3, (24000,), "tiled",
     dict(window=(5000,), sinks=(7,), softcap=(3.0,))),
    ("bf16-g8-q3-var", "bf16", 64, 16, 16, 2, 3, (24000, 3000), "split",
     dict(window=(64, 0), sinks=(3, 9), softcap=(0.0, 30.0))),
    ("f32-g4-q6-noncausal-alibi", "f32", 64, 64, 8, 2, 6, (12000,), "tiled",
     dict(causal=False, alibi=True, density=None)),
    ("bf16-g8-q7-mask", "bf16", 128, 16, 16, 2, 7, (20000, 5000), "tiled",
     dict(causal=True, alibi=False, density=0.5)),
    ("bf16-g4-q6-mask-alibi", "bf16", 64, 64, 8, 2, 6, (20000,), "split",
     dict(causal=True, alibi=True, density=0.95)),
    # one query position per workgroup (256 q-heads over one K/V head), with key splits
    ("bf16-g256-q2-keysplits", "bf16", 64, 256, 256, 1, 2, (66000,), "tiled", {}),
    ("f32-g256-q2-keysplits", "f32", 64, 64, 256, 1, 2, (33000,), "tiled", {}),
    # uneven head map: groups of 5, 3 and 1 q-heads, the largest sets the rows
    ("bf16-map5-q7", "bf16", 64, 16, 9, 3, 7, (20000,), "tiled", dict(head_map=[0, 1, 0, 2, 0, 1, 0, 0, 1])),
    ("bf16-map5-q6", "bf16", 64, 16, 9, 3, 6, (24000,), "split", dict(head_map=[0, 1, 0, 2, 0, 1, 0, 0, 1])),
    ("f32-map5-q2", "f32", 128, 64, 9, 3, 2, (33000,), "tiled", dict(head_map=[0, 1, 0, 2, 0, 1, 0, 0, 1])),
    # one query through the prefill entry: tiled from 2^17 pairs for either dtype
    ("bf16-g64-q1", "bf16", 128, 64, 64, 1, 1, (70000, 70000), "tiled", {}),
    ("bf16-g64-q1-small", "bf16", 64, 64, 64, 1, 1, (32768, 32768), "split", {}),
    ("f32-g32-q1", "f32", 64, 128, 32, 1, 1, (70000, 70000), "tiled", {}),
    ("f32-g32-q1-small", "f32", 64, 16, 32, 1, 1, (32768, 32768), "split", {}),
    ("bf16-g48-q1-var", "bf16", 128, 16, 48, 1, 1, (140000,), "tiled",
     dict(window=(30000,), sinks=(3,), softcap=(20.0,))),
]


@pytest.mark.parametrize("c", CASES, ids=[c[0] for c in CASES])
def test_short_query_block_matches_oracle(c, capfd, monkeypatch):
    name, dt, d, page, hq, hkv, q_len, lens, route, ex = c
    print(f"[short-tiled] {name} lens={lens}", flush=True)
    w = workloads.Workload(f"short_{name}", seed=900 + CASES.index(c), batch=len(lens), hq=hq, hkv=hkv,
                           head_dim=d, page_size=page, dtype=dt, q_len=q_len,
                           context_lens=np.asarray(lens, np.int32), scale=1.0 / math.sqrt(d), shuffle_pages=True)
    if "window" in ex:
        w.window = np.asarray(ex["window"], np.int32)
        w.sinks = np.asarray(ex["sinks"], np.int32)
        w.softcap = np.asarray(ex["softcap"], np.float32)
    inp = H.build(w, poison=True)
    capfd.readouterr()
    monkeypatch.setenv("ATLAS_DEBUG", "1")
    if "causal" in ex:
        slopes = alibi_slopes(w.hq) if ex["alibi"] else None
        mask = None
        if ex["density"]:
            L = int(w.page_size * ((int(w.context_lens.max()) + w.page_size - 1) // w.page_size))
            mask = np.random.default_rng(31 + q_len).random((w.batch, w.q_len, L)) < ex["density"]
            for b in range(w.batch):
                mask[b, np.arange(w.q_len), int(w.context_lens[b]) - w.q_len + np.arange(w.q_len)] = True
        out, lse = run_mods(inp, ex["causal"], slopes, mask)
    else:
        out, lse = H.run(inp, entry="prefill", head_map=ex.get("head_map"))
    torch.cuda.synchronize()
    monkeypatch.delenv("ATLAS_DEBUG")
    err = capfd.readouterr().err
    print(err.strip(), flush=True)
    want = "atlas: tiled prefill" if route == "tiled" else "atlas: split-KV prefill"
    assert want in err, f"{name}: expected the {route} kernels, stderr: {err!r}"
    if "causal" in ex:
        check_mods(inp, out, lse, ex["causal"], slopes, mask, name)
    else:
        H.check_against_oracle(inp, out, lse, head_map=ex.get("head_map"), what=name)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_decode_entry_keeps_split_kernels(dt, capfd, monkeypatch):
    """The shape that the prefill entry runs tiled (one query, 64 or 32
    q-heads over one K/V head, 2 x 70000 keys) runs the split-KV kernels
    through the decode entry; both match the oracle."""
    hq = 64 if dt == "bf16" else 32
    w = workloads.Workload(f"short_decode_{dt}", seed=880, batch=2, hq=hq, hkv=1, head_dim=64, page_size=64,
                           dtype=dt, q_len=1, context_lens=np.asarray((70000, 70000), np.int32), scale=0.125,
                           shuffle_pages=True)
    print(f"[short-tiled] decode entry {dt}", flush=True)
    inp = H.build(w, poison=True)
    capfd.readouterr()
    monkeypatch.setenv("ATLAS_DEBUG", "1")
    out_d, lse_d = H.run(inp, entry="decode")
    out_p, lse_p = H.run(inp, entry="prefill")
    torch.cuda.synchronize()
    monkeypatch.delenv("ATLAS_DEBUG")
    err = capfd.readouterr().err
    print(err.strip(), flush=True)
    lines = err.strip().splitlines()
    assert "atlas: split-KV decode" in lines[0] and "atlas: tiled prefill" in lines[1], err
    H.check_against_oracle(inp, out_d, lse_d, what=f"decode entry {dt}")
    H.check_against_oracle(inp, out_p, lse_p, what=f"prefill entry {dt}")

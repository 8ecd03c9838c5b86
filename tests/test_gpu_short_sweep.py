"""Seeded randomized GPU parity sweep of short query blocks (1 to 63 queries
per sequence) through the prefill and mods entries, where the dispatch picks
the tiled or the split-KV kernels by the rows of a K/V head (queries x
group) and the call's size: GQA groups 1 to 32, contexts of up to 40000 keys
(so calls on both sides of the size bound), bf16 and fp32, head dims 64 and
128, pages of 1 to 256 tokens, plain calls, per-sequence window / sink /
softcap variants and modifications (non-causal rows, ALiBi slopes, random
mask bits).  Every query row of a seeded subset of q-heads (the first, the
last and up to six more) is checked against the oracle.  40 configurations
drawn once from a fixed seed, NaN-poisoned arenas; each case prints itself
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


def draw_cases(seed=20261203, n=40):
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        hkv = int(rng.choice([1, 2, 4]))
        group = int(rng.choice([1, 2, 4, 8, 16, 32]))
        q_len = int(rng.choice([1, 2, 3, 5, 8, 12, 17, 24, 33, 48, 63]))
        batch = int(rng.integers(1, 4))
        lens = tuple(int(x) for x in rng.integers(q_len, q_len + 40000, size=batch))
        kind = str(rng.choice(["plain", "var", "mods"], p=[0.5, 0.25, 0.25]))
        c = dict(k=k, dtype=str(rng.choice(["bf16", "f32"])), d=int(rng.choice([64, 128])),
                 page=int(rng.choice([1, 16, 64, 256])), hkv=hkv, hq=hkv * group, q_len=q_len, lens=lens,
                 kind=kind, rseed=int(rng.integers(0, 1 << 30)))
        if kind == "var":
            c["window"] = tuple(int(x) for x in rng.choice([0, 64, 700, 5000], size=batch))
            c["sinks"] = tuple(int(x) for x in rng.integers(0, 70, size=batch))
            c["softcap"] = tuple(float(x) for x in rng.choice([0.0, 3.0, 50.0], size=batch))
        if kind == "mods":
            c["causal"] = bool(rng.random() < 0.5)
            c["alibi"] = bool(rng.random() < 0.6)
            c["density"] = [None, 0.5, 0.95][int(rng.integers(0, 3))]
            if c["causal"] and not c["alibi"] and c["density"] is None:
                c["alibi"] = True      # keep every mods case a real modification
        hq = c["hq"]
        extra = rng.choice(np.arange(1, max(hq - 1, 1)), size=min(6, max(hq - 2, 0)), replace=False) if hq > 2 else []
        c["heads"] = tuple(sorted({0, hq - 1, *(int(x) for x in extra)}))
        cases.append(c)
    return cases


CASES = draw_cases()


def case_id(c):
    return (f"{c['k']}-{c['kind']}-{c['dtype']}-d{c['d']}-p{c['page']}-h{c['hq']}x{c['hkv']}-q{c['q_len']}"
            f"-L{max(c['lens'])}")


@pytest.mark.parametrize("c", CASES, ids=case_id)
def test_short_sweep_matches_oracle(c):
    print(f"[short-sweep] {case_id(c)} lens={c['lens']} heads={c['heads']}", flush=True)
    w = workloads.Workload(f"short_sweep{c['k']}", seed=1700 + c["k"], batch=len(c["lens"]), hq=c["hq"],
                           hkv=c["hkv"], head_dim=c["d"], page_size=c["page"], dtype=c["dtype"], q_len=c["q_len"],
                           context_lens=np.asarray(c["lens"], np.int32), scale=1.0 / math.sqrt(c["d"]),
                           shuffle_pages=True)
    if c["kind"] == "var":
        w.window = np.asarray(c["window"], np.int32)
        w.sinks = np.asarray(c["sinks"], np.int32)
        w.softcap = np.asarray(c["softcap"], np.float32)
    inp = H.build(w, poison=True)
    heads = list(c["heads"])
    if c["kind"] == "mods":
        slopes = alibi_slopes(w.hq) if c["alibi"] else None
        mask = None
        if c["density"]:
            L = int(w.page_size * ((int(w.context_lens.max()) + w.page_size - 1) // w.page_size))
            mask = np.random.default_rng(c["rseed"]).random((w.batch, w.q_len, L)) < c["density"]
            for b in range(w.batch):
                mask[b, np.arange(w.q_len), int(w.context_lens[b]) - w.q_len + np.arange(w.q_len)] = True
        out, lse = run_mods(inp, c["causal"], slopes, mask)
        torch.cuda.synchronize()
        check_mods(inp, out, lse, c["causal"], slopes, mask, case_id(c), heads=heads)
    else:
        out, lse = H.run(inp, entry="prefill")
        torch.cuda.synchronize()
        H.check_against_oracle(inp, out, lse, heads=heads, what=case_id(c))

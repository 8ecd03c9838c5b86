"""Seeded randomized GPU parity sweep of the tiled prefills at larger sizes:
64 to 2048 queries over contexts of up to about 20000 keys, bf16 and fp32,
head dims 64 and 128, pages of 1 to 256 tokens, GQA ratios 1 to 8, plain
causal calls, per-sequence window / sink / softcap variants, and the
modifications (non-causal rows, ALiBi slopes, random mask bits).  The oracle
checks 48 random rows and the last 16 of every sequence, for every q-head.
40 configurations drawn once from a fixed seed, run through the C ABI on
NaN-poisoned arenas; each case prints itself first."""
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


def draw_cases(seed=20261206, n=40):
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        hkv = int(rng.choice([1, 2, 4, 8]))
        group = int(rng.choice([1, 2, 4, 8]))
        q_len = int(rng.choice([64, 200, 512, 1000, 2048]))
        batch = int(rng.integers(1, 3))
        lens = tuple(int(x) for x in rng.integers(q_len, q_len + 18000, size=batch))
        kind = str(rng.choice(["plain", "var", "mods"], p=[0.4, 0.3, 0.3]))
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
        cases.append(c)
    return cases


CASES = draw_cases()


def case_id(c):
    return (f"{c['k']}-{c['kind']}-{c['dtype']}-d{c['d']}-p{c['page']}-h{c['hq']}x{c['hkv']}-q{c['q_len']}"
            f"-L{max(c['lens'])}")


@pytest.mark.parametrize("c", CASES, ids=case_id)
def test_tiled_sweep_matches_oracle(c):
    print(f"[tiled-sweep] {case_id(c)} lens={c['lens']}", flush=True)
    w = workloads.Workload(f"tiled_sweep{c['k']}", seed=700 + c["k"], batch=len(c["lens"]), hq=c["hq"],
                           hkv=c["hkv"], head_dim=c["d"], page_size=c["page"], dtype=c["dtype"], q_len=c["q_len"],
                           context_lens=np.asarray(c["lens"], np.int32), scale=1.0 / math.sqrt(c["d"]),
                           shuffle_pages=True)
    if c["kind"] == "var":
        w.window = np.asarray(c["window"], np.int32)
        w.sinks = np.asarray(c["sinks"], np.int32)
        w.softcap = np.asarray(c["softcap"], np.float32)
    inp = H.build(w, poison=True)
    rng = np.random.default_rng(c["rseed"])
    rows = np.unique(np.concatenate([rng.choice(c["q_len"], size=min(48, c["q_len"]), replace=False),
                                     np.arange(max(0, c["q_len"] - 16), c["q_len"])]))
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
        check_mods(inp, out, lse, c["causal"], slopes, mask, case_id(c), rows=rows)
    else:
        out, lse = H.run(inp, entry="prefill")
        torch.cuda.synchronize()
        H.check_against_oracle(inp, out, lse, rows=rows, what=case_id(c))

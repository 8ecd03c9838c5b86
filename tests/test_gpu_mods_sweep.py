"""Seeded randomized GPU parity sweep of atlas_attend_mods on the tiled
prefill kernels (q_len >= 64), bf16 and fp32, with block-structured masks:
packed documents of random lengths, key blocks dropped for every row, and
stripes of blocks.  Such masks hide whole 64-key blocks from every row of a
query block, so the kernels' block lists drop them and mark the blocks every
row sees whole, which random element masks almost never do.  ALiBi on or
off, causal or non-causal rows, pages of 1 to 128 tokens (so that the
page-id window follows the outward ALiBi walk), a few rows that see nothing
(NaN with lse = -inf).  60 configurations drawn once from a fixed seed, each
run through the C ABI on NaN-poisoned arenas and checked against the fp64
oracle; each case prints itself first."""
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


def draw_cases(seed=20261205, n=60):
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        hkv = int(rng.choice([1, 2, 4]))
        group = int(rng.choice([1, 2, 4, 8]))
        batch = int(rng.integers(1, 3))
        q_len = int(rng.choice([64, 100, 257, 600]))
        lens = tuple(int(x) for x in rng.integers(q_len, q_len + 3000, size=batch))
        cases.append(dict(k=k, dtype=str(rng.choice(["bf16", "f32"])), d=int(rng.choice([64, 128])),
                          page=int(rng.choice([1, 2, 16, 128])), hkv=hkv, hq=hkv * group, q_len=q_len, lens=lens,
                          causal=bool(rng.random() < 0.6), alibi=bool(rng.random() < 0.5),
                          mtype=str(rng.choice(["doc", "blocks", "stripes"])),
                          mseed=int(rng.integers(0, 1 << 30))))
    return cases


CASES = draw_cases()


def case_id(c):
    return (f"{c['k']}-{c['dtype']}-d{c['d']}-p{c['page']}-h{c['hq']}x{c['hkv']}-q{c['q_len']}-L{max(c['lens'])}-"
            f"{'c' if c['causal'] else 'nc'}{'-alibi' if c['alibi'] else ''}-{c['mtype']}")


def structured_mask(c, w):
    """[B][q_len][L] keep-mask: documents of 20-399 tokens (a row sees its own
    document), 64-key blocks dropped with probability 0.4 (and 10 % of the
    remaining elements), or every m-th block dropped; each row keeps its own
    position, and in a fifth of the cases the first few rows see nothing."""
    rng = np.random.default_rng(c["mseed"])
    L = int(w.page_size * ((int(w.context_lens.max()) + w.page_size - 1) // w.page_size))
    j = np.arange(L)[None, :]
    m = np.zeros((w.batch, w.q_len, L), bool)
    for b in range(w.batch):
        pos = (int(w.context_lens[b]) - w.q_len + np.arange(w.q_len))[:, None]
        if c["mtype"] == "doc":
            bounds = np.cumsum(rng.integers(20, 400, size=L // 20 + 2))
            doc = np.searchsorted(bounds, np.arange(L), side="right")
            keep = doc[None, :] == doc[pos[:, 0]][:, None]
        elif c["mtype"] == "blocks":
            drop = rng.random(L // 64 + 1) < 0.4
            keep = ~drop[j // 64] & (rng.random((w.q_len, L)) < 0.9)
        else:
            mod = int(rng.integers(2, 5))
            r = int(rng.integers(0, mod))
            keep = np.broadcast_to((j // 64) % mod != r, (w.q_len, L)).copy()
        keep |= j == pos
        if rng.random() < 0.2:
            keep[: int(rng.integers(1, 8))] = False
        m[b] = keep
    return m


@pytest.mark.parametrize("c", CASES, ids=case_id)
def test_structured_masks_match_oracle(c):
    print(f"[mods-sweep] {case_id(c)} lens={c['lens']}", flush=True)
    w = workloads.Workload(f"mods_sweep{c['k']}", seed=500 + c["k"], batch=len(c["lens"]), hq=c["hq"],
                           hkv=c["hkv"], head_dim=c["d"], page_size=c["page"], dtype=c["dtype"], q_len=c["q_len"],
                           context_lens=np.asarray(c["lens"], np.int32), scale=1.0 / math.sqrt(c["d"]),
                           shuffle_pages=True)
    inp = H.build(w, poison=True, extra_phys=2)
    slopes = alibi_slopes(w.hq) if c["alibi"] else None
    mask = structured_mask(c, w)
    out, lse = run_mods(inp, c["causal"], slopes, mask)
    torch.cuda.synchronize()
    check_mods(inp, out, lse, c["causal"], slopes, mask, case_id(c))

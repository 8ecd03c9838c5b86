"""Seeded synthetic workloads: shapes, lengths, page layouts and random tensors.

This module is shared by the tests, the smoke check and the benchmark.  It
holds none of the attention arithmetic and none of the K/V regenerator: it
only draws sizes, page permutations, hot/cold splits and random-normal input
tensors from fixed seeds, so that the HIP path and the CPU oracle see the same
inputs.  Regenerated K/V values are NOT produced here; each side derives them
from the seed on its own.

Five workloads, named by what they are:

  single_head_decode   1 query, D=64, 4096-token context in 8 pages of 512,
                       fp32, K/V regenerated from seed (layer 0, head 0),
                       pages contiguous in order.
  gqa_short_query      B=1, Hq=8, Hkv=2, 16 queries as the suffix of a
                       256-token context, D=64, fp32, scale 0.125, pages of 64
                       (the CPUAttn README's parallel example).
  long_context_decode  B=8 x 65536 tokens, Hq=32, Hkv=8, D=64, pages of 512,
                       fp32, shuffled physical pool, 25 % of pages resident,
                       the rest regenerated into scratch on every call.
  causal_prefill       B=1, S=8192, Hq=32, Hkv=8, D=128, bf16, pages of 128
                       in a random physical order, scale 1/sqrt(128).
  mixed_decode         B=64, lengths uniform in [1024, 32768], Hq=64, Hkv=8,
                       D=128, pages of 16, bf16 Q/K/V, shuffled pool; even
                       sequences use window 4096 + 4 sink tokens + softcap 50,
                       odd ones plain causal.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

WORKLOADS = ("single_head_decode", "gqa_short_query", "long_context_decode",
             "causal_prefill", "mixed_decode")


@dataclass
class Workload:
    name: str
    seed: int
    batch: int
    hq: int
    hkv: int
    head_dim: int
    page_size: int
    dtype: str                     # "f32" or "bf16" (K/V, and Q unless q_dtype says otherwise)
    q_len: int                     # 1 for decode
    context_lens: np.ndarray       # [B] int32
    scale: float
    regenerated: bool = False      # K/V come from the seeded regenerator
    hot_fraction: float = 1.0      # share of pages kept resident (regenerated workloads)
    shuffle_pages: bool = True
    window: np.ndarray | None = None     # [B] int32, 0 = off
    sinks: np.ndarray | None = None      # [B] int32
    softcap: np.ndarray | None = None    # [B] float32, 0 = off
    layer: int = 0
    q_dtype: str | None = None           # Q's dtype when it differs from the K/V dtype
    seq_keys: np.ndarray | None = None   # [B] generator keys of regenerated sequences (None: the batch row)
    extra: dict = field(default_factory=dict)

    @property
    def qdt(self) -> str:
        return self.q_dtype or self.dtype

    def seq_key(self, b: int) -> int:
        return int(b if self.seq_keys is None else self.seq_keys[b])

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def max_pages(self) -> int:
        return int(max(1, math.ceil(int(self.context_lens.max()) / self.page_size)))


def make(name: str, **overrides) -> Workload:
    """The named workload at its full size (overrides allow reduced variants)."""
    if name == "single_head_decode":
        w = Workload(name, seed=1, batch=1, hq=1, hkv=1, head_dim=64, page_size=512, dtype="f32",
                     q_len=1, context_lens=np.array([4096], np.int32), scale=1.0 / 8.0,
                     regenerated=True, hot_fraction=1.0, shuffle_pages=False)
    elif name == "gqa_short_query":
        w = Workload(name, seed=2, batch=1, hq=8, hkv=2, head_dim=64, page_size=64, dtype="f32",
                     q_len=16, context_lens=np.array([256], np.int32), scale=0.125,
                     shuffle_pages=False)
    elif name == "long_context_decode":
        w = Workload(name, seed=3, batch=8, hq=32, hkv=8, head_dim=64, page_size=512, dtype="f32",
                     q_len=1, context_lens=np.full(8, 65536, np.int32), scale=1.0 / 8.0,
                     regenerated=True, hot_fraction=0.25, shuffle_pages=True)
    elif name == "causal_prefill":
        w = Workload(name, seed=4, batch=1, hq=32, hkv=8, head_dim=128, page_size=128,
                     dtype="bf16", q_len=8192, context_lens=np.array([8192], np.int32),
                     scale=1.0 / math.sqrt(128.0), shuffle_pages=True)
    elif name == "mixed_decode":
        rng = np.random.default_rng(5)
        lens = rng.integers(1024, 32768, size=64, endpoint=True).astype(np.int32)
        even = (np.arange(64) % 2 == 0)
        w = Workload(name, seed=5, batch=64, hq=64, hkv=8, head_dim=128, page_size=16,
                     dtype="bf16", q_len=1, context_lens=lens, scale=1.0 / math.sqrt(128.0),
                     shuffle_pages=True,
                     window=np.where(even, 4096, 0).astype(np.int32),
                     sinks=np.where(even, 4, 0).astype(np.int32),
                     softcap=np.where(even, 50.0, 0.0).astype(np.float32))
    else:
        raise KeyError(name)
    for k, v in overrides.items():
        setattr(w, k, v)
    return w


# ------------------------------------------------------------ page layout

@dataclass
class PageLayout:
    """Physical placement of every logical page.

    page_table[b][p] is the physical page id of logical page p of sequence b
    (entries past a sequence's last page are 0 and never read).  For
    regenerated workloads ids [0, n_hot) form the resident pool and ids
    [n_hot, n_hot + n_cold) the scratch region; `cold_jobs` lists
    (batch row, logical_page, phys_page) for every cold page and `hot_jobs`
    the same for resident pages (filled once, before any timed call);
    `key_jobs` turns such a list into regeneration jobs, whose first column is
    the sequence's generator key."""
    page_table: np.ndarray          # [B][max_pages] int32
    num_phys: int
    hot_jobs: np.ndarray            # [n][3] int32
    cold_jobs: np.ndarray           # [n][3] int32


def key_jobs(w: Workload, jobs: np.ndarray) -> np.ndarray:
    """(batch row, logical page, phys page) -> (generator key, logical page, phys page)."""
    out = np.array(jobs, np.int32).reshape(-1, 3).copy()
    if w.seq_keys is not None and len(out):
        out[:, 0] = np.asarray(w.seq_keys, np.int32)[out[:, 0]]
    return out


def page_layout(w: Workload, hot_fraction: float | None = None, seed_offset: int = 0,
                extra_phys: int = 0) -> PageLayout:
    """Seeded placement: per-sequence page counts from the context lengths, a
    shuffled (or in-order) physical assignment, and for regenerated workloads a
    seeded hot subset of each sequence's pages.  `extra_phys` appends unused
    physical pages (poison targets in tests)."""
    rng = np.random.default_rng(1000 + w.seed + seed_offset)
    hf = w.hot_fraction if hot_fraction is None else hot_fraction
    P = w.page_size
    n_pages = [int(math.ceil(int(L) / P)) for L in w.context_lens]
    maxp = max(n_pages)
    pt = np.zeros((w.batch, maxp), np.int32)
    logical = [(b, p) for b in range(w.batch) for p in range(n_pages[b])]
    total = len(logical)
    if w.regenerated:
        hot = np.zeros(total, bool)
        start = 0
        for b in range(w.batch):
            k = int(round(hf * n_pages[b]))
            pick = rng.choice(n_pages[b], size=k, replace=False) if k > 0 else np.array([], int)
            hot[start + pick] = True
            start += n_pages[b]
        n_hot = int(hot.sum())
        hot_ids = rng.permutation(n_hot) if w.shuffle_pages else np.arange(n_hot)
        cold_ids = n_hot + (rng.permutation(total - n_hot) if w.shuffle_pages
                            else np.arange(total - n_hot))
        hj, cj = [], []
        hi = ci = 0
        for idx, (b, p) in enumerate(logical):
            if hot[idx]:
                pid = int(hot_ids[hi]); hi += 1
                hj.append((b, p, pid))
            else:
                pid = int(cold_ids[ci]); ci += 1
                cj.append((b, p, pid))
            pt[b, p] = pid
        hot_jobs = np.array(hj, np.int32).reshape(-1, 3)
        cold_jobs = np.array(cj, np.int32).reshape(-1, 3)
    else:
        ids = rng.permutation(total) if w.shuffle_pages else np.arange(total)
        for idx, (b, p) in enumerate(logical):
            pt[b, p] = int(ids[idx])
        hot_jobs = np.zeros((0, 3), np.int32)
        cold_jobs = np.zeros((0, 3), np.int32)
    return PageLayout(pt, total + extra_phys, hot_jobs, cold_jobs)


# ---------------------------------------------------------- random tensors

def randn(shape, seed: int, dtype: str = "f32", device: str = "cpu"):
    """Seeded N(0,1) tensor (torch), drawn in fp32 and rounded to `dtype`
    ("f32" or "bf16", round-to-nearest-even).  The same (seed, device) always
    gives the same bits."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(tuple(int(s) for s in shape), generator=g, device=device, dtype=torch.float32)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype != "f32":
        raise ValueError(dtype)
    return t


def logical_kv(w: Workload, device: str = "cpu", seed_offset: int = 0):
    """Seeded K/V in logical page order: [total_pages][Hkv][P][D] (pages of
    sequence 0 first), independent of any physical placement.  Used by the
    workloads whose K/V are not regenerated."""
    n_pages = [int(math.ceil(int(L) / w.page_size)) for L in w.context_lens]
    shape = (sum(n_pages), w.hkv, w.page_size, w.head_dim)
    k = randn(shape, seed=w.seed * 100 + 2 + seed_offset, dtype=w.dtype, device=device)
    v = randn(shape, seed=w.seed * 100 + 3 + seed_offset, dtype=w.dtype, device=device)
    return k, v, n_pages


def query_shape(w: Workload):
    return (w.batch, w.q_len, w.hq, w.head_dim)


def arena_shape(w: Workload, num_phys: int):
    return (num_phys, w.hkv, w.page_size, w.head_dim)


"""GPU parity at the largest sizes the library accepts (include/atlas.h):
256 q-heads over one K/V head (a group of 256: one query position per tiled
workgroup), 256 K/V heads (multi-head attention), pages of 4096 tokens, on
the decode, the tiled prefills (bf16 and fp32), their key splits, the
short-query split path and atlas_attend_mods, against the oracle on
NaN-poisoned arenas.  Each case prints itself first."""
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


def say(*a):
    print(*a, flush=True)


def wl(dtype, hq, hkv, d, page, q_len, lens, seed):
    return workloads.Workload("limits", seed=seed, batch=len(lens), hq=hq, hkv=hkv, head_dim=d, page_size=page,
                              dtype=dtype, q_len=q_len, context_lens=np.asarray(lens, np.int32),
                              scale=1.0 / math.sqrt(d), shuffle_pages=True)


CASES = [
    # (dtype, hq, hkv, d, page, q_len, lens)
    ("f32", 256, 1, 64, 4096, 1, (5000, 4097, 1)),       # decode, group of 256, largest pages
    ("bf16", 256, 256, 128, 16, 1, (300, 77)),           # decode, 256 K/V heads
    ("bf16", 256, 1, 128, 4096, 70, (70, 5000)),         # tiled bf16 prefill, one position per workgroup
    ("f32", 128, 2, 64, 4096, 100, (100, 4500)),         # tiled fp32 prefill, group of 64
    ("bf16", 256, 256, 128, 64, 16, (16, 900)),          # short-query split path, 256 K/V heads
    ("bf16", 64, 1, 128, 4096, 64, (20000,)),            # tiled bf16 prefill with key splits
    ("f32", 64, 1, 64, 4096, 64, (20000,)),              # tiled fp32 prefill with key splits
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-h{c[1]}x{c[2]}-d{c[3]}-p{c[4]}-q{c[5]}")
def test_limits_match_oracle(case):
    dtype, hq, hkv, d, page, q_len, lens = case
    say(f"[limits] {case}")
    w = wl(dtype, hq, hkv, d, page, q_len, lens, seed=70 + hq + hkv + page)
    inp = H.build(w, poison=True, extra_phys=1)
    out, lse = H.run(inp)
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what=str(case))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_limits_mods(dtype):
    """256 q-heads over one K/V head with non-causal rows and ALiBi slopes
    on the tiled path (pages of 4096)."""
    w = wl(dtype, 256, 1, 64, 4096, 64, (64, 3000), seed=91)
    say(f"[limits] mods {dtype} h256x1 p4096 q64 non-causal ALiBi")
    inp = H.build(w, poison=True)
    slopes = alibi_slopes(256)
    out, lse = run_mods(inp, False, slopes, None)
    torch.cuda.synchronize()
    check_mods(inp, out, lse, False, slopes, None, f"limits mods {dtype}")

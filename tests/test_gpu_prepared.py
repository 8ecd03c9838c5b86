"""Prepared calls (prepare_attend): the arguments are checked and marshalled
once and each call only re-issues the C-ABI call.  They must give the same
bits as the ordinary binding calls on the same tensors, also after the
tensors' contents change between calls (new queries, shorter lengths,
pages swapped in the page table), for decode and prefill, fp32 and bf16.
Each test prints its case first."""
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


@pytest.mark.parametrize("dtype,q_len,lens", [("f32", 1, (4096, 300, 9)), ("bf16", 1, (2000, 150)),
                                              ("f32", 16, (256,)), ("bf16", 100, (700, 900))])
def test_prepared_call_equals_the_ordinary_call(dtype, q_len, lens):
    import exact_paged_causal_amd as atlas
    print(f"[prepared] {dtype} q_len={q_len} lens={lens}", flush=True)
    d = 64 if dtype == "f32" else 128
    w = workloads.Workload("prepared", seed=71, batch=len(lens), hq=8, hkv=2, head_dim=d, page_size=16, dtype=dtype,
                           q_len=q_len, context_lens=np.asarray(lens, np.int32), scale=1.0 / math.sqrt(d),
                           shuffle_pages=True)
    inp = H.build(w, extra_phys=4)
    kind = "decode" if q_len == 1 else "prefill"
    plain = atlas.atlas_attend_decode if kind == "decode" else atlas.atlas_attend_prefill
    q = inp.q.clone()
    pt = inp.page_table.clone()
    ctx = inp.context_lens.clone()
    out = torch.empty(w.batch, q_len, w.hq, d, dtype=torch.float32, device="cuda")
    lse = torch.empty(w.batch, q_len, w.hq, dtype=torch.float32, device="cuda")
    call = atlas.prepare_attend(kind, q, inp.k, inp.v, pt, ctx, w.scale, out=out, lse=lse)
    for step in range(3):
        o, l = call()
        assert o is out and l is lse
        ref_o, ref_l = plain(q, inp.k, inp.v, pt, ctx, w.scale)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), step
        # new contents for the next call: queries, a shorter first context,
        # two pages of the first sequence swapped in the page table
        q.copy_(torch.roll(q, 1, dims=-1))
        ctx[0] = max(q_len, int(ctx[0]) - 7)
        n0 = (int(ctx[0]) + w.page_size - 1) // w.page_size
        if n0 >= 2:
            a, b = pt[0, 0].item(), pt[0, n0 - 1].item()
            pt[0, 0], pt[0, n0 - 1] = b, a

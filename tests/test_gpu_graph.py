"""Decode and short prefill calls captured in a HIP graph (torch.cuda.CUDAGraph)
and replayed.  Outside validation mode a call is kernel launches only (no
allocation, copy, memset or synchronisation), so it can be captured; the
graph is replayed several times with eager work and synchronisations in
between, the inputs' contents changed before each replay, and every replay
is compared bit for bit with the same call made eagerly.  Each test prints
its case first."""
import math
import os

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


@pytest.mark.parametrize("dtype,q_len,lens", [("f32", 1, (4096,)), ("bf16", 1, (3000, 700, 40)),
                                              ("f32", 16, (256, 90)), ("bf16", 1, (200,))])
def test_graph_replays_equal_eager_calls(dtype, q_len, lens):
    import exact_paged_causal_amd as atlas
    if os.environ.get("ATLAS_VALIDATE", "") not in ("", "0"):
        pytest.skip("validation mode copies device arrays to the host and synchronises: not capturable")
    print(f"[graph] {dtype} q_len={q_len} lens={lens}", flush=True)
    d = 64 if dtype == "f32" else 128
    w = workloads.Workload("graph", seed=73, batch=len(lens), hq=8, hkv=2, head_dim=d, page_size=64, dtype=dtype,
                           q_len=q_len, context_lens=np.asarray(lens, np.int32), scale=1.0 / math.sqrt(d),
                           shuffle_pages=True)
    inp = H.build(w)
    kind = "decode" if q_len == 1 else "prefill"
    eager = atlas.atlas_attend_decode if kind == "decode" else atlas.atlas_attend_prefill
    q = inp.q.clone()
    ctx = inp.context_lens.clone()
    out = torch.empty(w.batch, q_len, w.hq, d, dtype=torch.float32, device="cuda")
    lse = torch.empty(w.batch, q_len, w.hq, dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        call = atlas.prepare_attend(kind, q, inp.k, inp.v, inp.page_table, ctx, w.scale, out=out, lse=lse)
        call()                                   # eager first call on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call()
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    for rep in range(4):
        # new contents, then eager work of the program's own between replays
        q.copy_(torch.randn(q.shape, generator=gen, device="cuda", dtype=torch.float32).to(q.dtype))
        ctx[0] = max(q_len, int(lens[0]) - 13 * rep)
        scratch = torch.randn(1 << 16, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        ref_o, ref_l = eager(q, inp.k, inp.v, inp.page_table, ctx, w.scale)
        torch.cuda.synchronize()
        assert torch.equal(got_o, ref_o) and torch.equal(got_l, ref_l), f"replay {rep}"
        assert torch.isfinite(scratch)


def test_graph_of_the_allocation_free_decode():
    """atlas_attend_decode_noalloc, whose callers are the ones that cannot
    allocate (graph capture among them), captured after one eager call on
    the capture stream (which looks up the library's array) and replayed
    with new queries and lengths: every replay equals the workspace decode
    bit for bit."""
    import exact_paged_causal_amd as atlas
    if os.environ.get("ATLAS_VALIDATE", "") not in ("", "0"):
        pytest.skip("the allocation-free decode refuses validation mode")
    print("[graph] allocation-free decode", flush=True)
    w = workloads.Workload("graph_noalloc", seed=74, batch=3, hq=16, hkv=4, head_dim=128, page_size=16,
                           dtype="bf16", q_len=1, context_lens=np.asarray([2500, 600, 77], np.int32),
                           scale=1.0 / math.sqrt(128), shuffle_pages=True)
    inp = H.build(w)
    q = inp.q.clone()
    ctx = inp.context_lens.clone()
    out = torch.empty(w.batch, 1, w.hq, 128, dtype=torch.float32, device="cuda")
    lse = torch.empty(w.batch, 1, w.hq, dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        atlas.atlas_attend_decode_noalloc(q, inp.k, inp.v, inp.page_table, ctx, w.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        atlas.atlas_attend_decode_noalloc(q, inp.k, inp.v, inp.page_table, ctx, w.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(6)
    for rep in range(3):
        q.copy_(torch.randn(q.shape, generator=gen, device="cuda", dtype=torch.float32).to(q.dtype))
        ctx[1] = 600 - 50 * rep
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        ref_o, ref_l = atlas.atlas_attend_decode(q, inp.k, inp.v, inp.page_table, ctx, w.scale)
        torch.cuda.synchronize()
        assert torch.equal(got_o, ref_o) and torch.equal(got_l, ref_l), f"replay {rep}"

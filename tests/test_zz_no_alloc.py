"""GPU test of atlas_attend_decode_noalloc, the decode entry point that
allocates nothing (its partial states live in the library's own 32 MiB
device array): through the C ABI, its outputs equal atlas_attend_decode's
bit for bit (hence within the fp32 / bf16 bars of the oracle as well) on
consecutive calls of decreasing size, so contents the previous call left in
the array never leak into the next.  Each test prints its case first."""
import ctypes
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


def say(*a):
    print(*a, flush=True)


def validation_mode():
    """The library's ATLAS_VALIDATE switch (set and not "0")."""
    v = os.environ.get("ATLAS_VALIDATE", "")
    return v not in ("", "0")


def noalloc(inp, out, lse):
    """One call through the C ABI with prepared outputs (nothing allocated).
    Validation mode copies device arrays to host buffers, which this entry
    point never does: there it must refuse with ATLAS_ERR_UNSUPPORTED."""
    from exact_paged_causal_amd import atlas
    w = inp.w
    args, keep = atlas.make_attn_args(inp.q, inp.k, inp.v, inp.page_table, inp.context_lens, w.scale,
                                      window=inp.window, sink_tokens=inp.sinks, softcap=inp.softcap,
                                      out=out, lse=lse)
    st = atlas.lib.atlas_attend_decode_noalloc(ctypes.byref(args),
                                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if validation_mode():
        assert st == atlas.ATLAS_ERR_UNSUPPORTED, atlas.atlas_last_error()
        pytest.skip("validation mode: the allocation-free decode refuses it (checked)")
    assert st == atlas.ATLAS_OK, atlas.atlas_last_error()


def reference(inp):
    import exact_paged_causal_amd as atlas
    w = inp.w
    return atlas.atlas_attend_decode(inp.q, inp.k, inp.v, inp.page_table, inp.context_lens, w.scale,
                                     window=inp.window, sink_tokens=inp.sinks, softcap=inp.softcap)


def outputs(w):
    return (torch.full((w.batch, 1, w.hq, w.head_dim), 7.0, device="cuda"),
            torch.full((w.batch, 1, w.hq), 7.0, device="cuda"))


def test_noalloc_equals_workspace_decode_on_shrinking_calls():
    import exact_paged_causal_amd as atlas
    # 1. the long-context decode (8 x 65536, fp32, 75 % regenerated): 2 MiB of partial states
    w1 = workloads.make("long_context_decode")
    say("[noalloc] long_context_decode (8 x 65536, fp32)")
    inp1 = H.build(w1)
    H.run(inp1)                                   # regenerates the cold pages into scratch pages
    ref_o1, ref_l1 = reference(inp1)
    o1, l1 = outputs(w1)
    noalloc(inp1, o1, l1)
    torch.cuda.synchronize()
    assert torch.equal(o1, ref_o1) and torch.equal(l1, ref_l1)
    # 2. a smaller bf16 decode with windows, sinks and softcap, right after
    w2 = workloads.Workload("noalloc_small", seed=61, batch=3, hq=8, hkv=2, head_dim=128, page_size=16,
                            dtype="bf16", q_len=1, context_lens=np.array([700, 33, 1500], np.int32),
                            scale=1.0 / math.sqrt(128), window=np.array([64, 0, 500], np.int32),
                            sinks=np.array([4, 0, 2], np.int32), softcap=np.array([30.0, 0.0, 5.0], np.float32))
    say("[noalloc] small bf16 decode with variants, after the large one")
    inp2 = H.build(w2)
    ref_o2, ref_l2 = reference(inp2)
    o2, l2 = outputs(w2)
    noalloc(inp2, o2, l2)
    torch.cuda.synchronize()
    assert torch.equal(o2, ref_o2) and torch.equal(l2, ref_l2)
    H.check_against_oracle(inp2, o2, l2, what="noalloc small bf16")
    # 3. the smallest: one sequence, one head, through the binding, without lse
    w3 = workloads.make("single_head_decode")
    say("[noalloc] single-head decode, no lse")
    inp3 = H.build(w3)
    ref_o3, _ = reference(inp3)
    o3 = torch.full((1, 1, 1, 64), 7.0, device="cuda")
    atlas.atlas_attend_decode_noalloc(inp3.q, inp3.k, inp3.v, inp3.page_table, inp3.context_lens, w3.scale, out=o3)
    torch.cuda.synchronize()
    assert torch.equal(o3, ref_o3)


def test_noalloc_rejects_oversized_and_validation(monkeypatch):
    import exact_paged_causal_amd as atlas
    say("[noalloc] partial states beyond the array; validation mode")
    w = workloads.Workload("noalloc_big", seed=62, batch=64, hq=64, hkv=8, head_dim=128, page_size=4096,
                           dtype="bf16", q_len=1, context_lens=np.full(64, 4096 * 16, np.int32),
                           scale=1.0 / math.sqrt(128))
    q = torch.zeros((64, 1, 64, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 8, 4096, 128), dtype=torch.bfloat16, device="cuda")
    pt = torch.zeros((64, 16), dtype=torch.int32, device="cuda")
    ctx = torch.from_numpy(w.context_lens).cuda()
    out = torch.full((64, 1, 64, 128), 7.0, device="cuda")
    with pytest.raises(atlas.AtlasError) as ei:
        atlas.atlas_attend_decode_noalloc(q, k, k, pt, ctx, w.scale, out=out, split_tokens=4096)
    assert ei.value.status == atlas.ATLAS_ERR_WORKSPACE
    monkeypatch.setenv("ATLAS_VALIDATE", "1")
    with pytest.raises(atlas.AtlasError) as ei:
        atlas.atlas_attend_decode_noalloc(q[:1], k, k, pt[:1, :1], ctx[:1] // 16, w.scale, out=out[:1])
    assert ei.value.status == atlas.ATLAS_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)

"""GPU parity of atlas_attend_decode_regen: decode with the cold pages
regenerated inside the attention kernel (page-table entries -1) instead of
into scratch pages.  Checked against the fp64 oracle and, bit for bit,
against regenerating the same pages into scratch and running
atlas_attend_decode.

Each test prints the case it runs before touching the GPU."""
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


def say(*a):
    print(*a, flush=True)


def fused_table(inp):
    """The build's page table with every cold page replaced by -1."""
    pt = inp.layout.page_table.copy()
    for seq, lp, _ in inp.layout.cold_jobs:
        pt[seq, lp] = -1
    return torch.from_numpy(pt).cuda()


def run_fused(inp, pt=None, **kw):
    import exact_paged_causal_amd as atlas
    w = inp.w
    return atlas.atlas_attend_decode_regen(inp.q, inp.k, inp.v, fused_table(inp) if pt is None else pt,
                                           inp.context_lens, w.scale, seed=w.seed, layer=w.layer,
                                           window=inp.window, sink_tokens=inp.sinks, softcap=inp.softcap, **kw)


def regen_workload(batch, lens, *, d=64, page=512, hq=32, hkv=8, hot=0.25, window=None, sinks=None,
                   softcap=None, seed=3):
    return workloads.Workload(
        "fused", seed=seed, batch=batch, hq=hq, hkv=hkv, head_dim=d, page_size=page, dtype="f32",
        q_len=1, context_lens=np.asarray(lens, np.int32), scale=1.0 / math.sqrt(d), regenerated=True,
        hot_fraction=hot, shuffle_pages=True,
        window=None if window is None else np.asarray(window, np.int32),
        sinks=None if sinks is None else np.asarray(sinks, np.int32),
        softcap=None if softcap is None else np.asarray(softcap, np.float32))


@pytest.mark.parametrize("case", [
    # (batch, lens, d, page, hq, hkv, hot)
    (3, (8192, 5000, 1), 64, 512, 32, 8, 0.25),
    (2, (300, 77), 64, 1, 8, 2, 0.5),        # one key per page: hot and cold keys inside one wave
    (2, (1000, 513), 128, 16, 8, 2, 0.3),    # 512-byte rows, two pieces per lane
    (1, (4096,), 64, 512, 1, 1, 0.0),        # single head, every page cold
], ids=lambda c: f"b{c[0]}-d{c[2]}-p{c[3]}-h{c[4]}x{c[5]}-hot{c[6]}")
def test_fused_matches_oracle_and_scratch_path(case):
    batch, lens, d, page, hq, hkv, hot = case
    w = regen_workload(batch, lens, d=d, page=page, hq=hq, hkv=hkv, hot=hot)
    say(f"[fused] {case}")
    # NaN everywhere the build does not write: the fused call must not read
    # the (still unregenerated) scratch pages of its cold pages.
    inp = H.build(w, poison=True)
    out_f, lse_f = run_fused(inp)
    torch.cuda.synchronize()
    assert not torch.isnan(out_f).any()
    H.check_against_oracle(inp, out_f, lse_f, what=f"fused {case}")
    say(f"[fused] scratch path {case}")
    out_s, lse_s = H.run(inp)          # regenerates the cold pages into scratch, then decodes
    torch.cuda.synchronize()
    assert torch.equal(out_f, out_s) and torch.equal(lse_f, lse_s)


def test_fused_with_window_sinks_softcap():
    w = regen_workload(3, (3000, 2500, 700), hq=8, hkv=2, page=64, hot=0.4,
                       window=(512, 0, 100), sinks=(4, 0, 2), softcap=(30.0, 0.0, 5.0))
    say("[fused] window / sinks / softcap")
    inp = H.build(w, poison=True)
    out_f, lse_f = run_fused(inp, split_tokens=1024)
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out_f, lse_f, what="fused variants")
    out_s, lse_s = H.run(inp, split_tokens=1024)
    torch.cuda.synchronize()
    assert torch.equal(out_f, out_s) and torch.equal(lse_f, lse_s)


def test_fused_long_context_full_size():
    """8 x 65536-token fp32 decode with the 75 % cold pages generated in the
    kernel: every (sequence, q-head) against the oracle, and bit-identical to
    the scratch path."""
    w = workloads.make("long_context_decode")
    say("[fused] long_context_decode full size")
    inp = H.build(w)
    out_f, lse_f = run_fused(inp)
    out_f, lse_f = out_f.clone(), lse_f.clone()
    out_s, lse_s = H.run(inp)
    torch.cuda.synchronize()
    assert torch.equal(out_f, out_s) and torch.equal(lse_f, lse_s)
    H.check_against_oracle(inp, out_f, lse_f, what="fused long_context_decode")


def test_fused_all_cold_single_head_equals_resident():
    w = workloads.make("single_head_decode")
    say("[fused] single head, resident vs generated in the kernel")
    res = H.build(w)
    out_r, lse_r = H.run(res)
    cold = H.build(workloads.make("single_head_decode", hot_fraction=0.0))
    out_f, lse_f = run_fused(cold)
    torch.cuda.synchronize()
    assert torch.equal(out_r, out_f) and torch.equal(lse_r, lse_f)


def test_fused_validation_mode(monkeypatch):
    import exact_paged_causal_amd as atlas
    monkeypatch.setenv("ATLAS_VALIDATE", "1")
    w = regen_workload(2, (900, 333), hq=4, hkv=2, page=64, hot=0.5)
    say("[fused] validation mode accepts -1 entries")
    inp = H.build(w)
    out_f, lse_f = run_fused(inp)
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out_f, lse_f, what="fused validated")
    say("[fused] validation mode rejects -2")
    pt = fused_table(inp)
    pt[1, 0] = -2
    with pytest.raises(atlas.AtlasError) as ei:
        run_fused(inp, pt=pt)
    assert ei.value.status == atlas.ATLAS_ERR_POOL

"""GPU parity of atlas_attend_decode_regen: decode with the cold pages
regenerated inside the attention kernel (page-table entries -1) instead of
into scratch pages, for fp32 and bf16 caches (the latter with bf16 or fp32
queries) and for explicit per-sequence generator keys.  Checked against the
fp64 oracle and, bit for bit, against regenerating the same pages into
scratch and running atlas_attend_decode.

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
                                           seq_keys=H.seq_keys_tensor(w),
                                           window=inp.window, sink_tokens=inp.sinks, softcap=inp.softcap, **kw)


def regen_workload(batch, lens, *, d=64, page=512, hq=32, hkv=8, hot=0.25, window=None, sinks=None,
                   softcap=None, seed=3, dtype="f32", q_dtype=None, seq_keys=None):
    return workloads.Workload(
        "fused", seed=seed, batch=batch, hq=hq, hkv=hkv, head_dim=d, page_size=page, dtype=dtype,
        q_len=1, context_lens=np.asarray(lens, np.int32), scale=1.0 / math.sqrt(d), regenerated=True,
        hot_fraction=hot, shuffle_pages=True, q_dtype=q_dtype,
        seq_keys=None if seq_keys is None else np.asarray(seq_keys, np.int32),
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


@pytest.mark.parametrize("case", [
    # (dtype, q_dtype, batch, lens, d, page, hq, hkv, hot)
    ("bf16", None, 3, (8192, 5000, 1), 128, 16, 16, 2, 0.25),
    ("bf16", None, 2, (300, 77), 128, 1, 8, 2, 0.5),      # one key per page: hot and cold rows in one chunk
    ("bf16", None, 2, (1000, 513), 64, 64, 8, 8, 0.3),
    ("bf16", "f32", 2, (2000, 700), 128, 16, 8, 1, 0.25),  # fp32 query over a bf16 cache
    ("bf16", None, 1, (4096,), 128, 512, 1, 1, 0.0),      # every page cold
], ids=lambda c: f"{c[0]}-q{c[1] or c[0]}-b{c[2]}-d{c[4]}-p{c[5]}-h{c[6]}x{c[7]}-hot{c[8]}")
def test_fused_bf16_matches_oracle_and_scratch_path(case):
    """bf16 caches: the fold builds cold keys' rows from the generator (each
    value rounded to bf16 as the regenerator stores it)."""
    dtype, qdt, batch, lens, d, page, hq, hkv, hot = case
    w = regen_workload(batch, lens, d=d, page=page, hq=hq, hkv=hkv, hot=hot, dtype=dtype, q_dtype=qdt)
    say(f"[fused bf16] {case}")
    inp = H.build(w, poison=True)
    out_f, lse_f = run_fused(inp)
    torch.cuda.synchronize()
    assert not torch.isnan(out_f).any()
    H.check_against_oracle(inp, out_f, lse_f, what=f"fused bf16 {case}")
    say(f"[fused bf16] scratch path {case}")
    out_s, lse_s = H.run(inp)
    torch.cuda.synchronize()
    assert torch.equal(out_f, out_s) and torch.equal(lse_f, lse_s)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_with_sequence_keys(dtype):
    """Explicit generator keys (one above 2^15, one 0): the cold pages come
    from each sequence's key, not its batch row, in the kernel and in the
    regenerator alike."""
    w = regen_workload(3, (1500, 900, 2100), d=64 if dtype == "f32" else 128, hq=8, hkv=2, page=64, hot=0.4,
                       dtype=dtype, seq_keys=(40000, 0, 7))
    say(f"[fused] sequence keys {dtype}")
    inp = H.build(w, poison=True)
    out_f, lse_f = run_fused(inp)
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out_f, lse_f, what=f"fused keys {dtype}")
    out_s, lse_s = H.run(inp)
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


def test_fused_bf16_mixed_decode_full_size():
    """The mixed-length bf16 decode (64 sequences, windows / sinks / softcap
    on the even ones) with K/V regenerated and 75 % of the pages generated in
    the kernel: bit-identical to the scratch path, and against the oracle on
    every sequence."""
    w = workloads.make("mixed_decode", regenerated=True, hot_fraction=0.25)
    say("[fused] mixed_decode full size, bf16, regenerated")
    inp = H.build(w)
    out_f, lse_f = run_fused(inp)
    out_f, lse_f = out_f.clone(), lse_f.clone()
    out_s, lse_s = H.run(inp)
    torch.cuda.synchronize()
    assert torch.equal(out_f, out_s) and torch.equal(lse_f, lse_s)
    # the oracle regenerates every row it reads on the CPU: the two shortest
    # windowed (even) and plain (odd) sequences
    order = np.argsort(w.context_lens, kind="stable")
    seqs = [int(b) for b in order if b % 2 == 0][:2] + [int(b) for b in order if b % 2 == 1][:2]
    H.check_against_oracle(inp, out_f, lse_f, seqs=seqs, what="fused mixed_decode")


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
    say("[fused] validation mode rejects a sequence key of 65536")
    keys = torch.tensor([3, 65536], dtype=torch.int32, device="cuda")
    with pytest.raises(atlas.AtlasError) as ei:
        atlas.atlas_attend_decode_regen(inp.q, inp.k, inp.v, fused_table(inp), inp.context_lens, w.scale,
                                        seed=w.seed, layer=w.layer, seq_keys=keys)
    assert ei.value.status == atlas.ATLAS_ERR_RANGE

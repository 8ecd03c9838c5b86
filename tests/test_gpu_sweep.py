"""Seeded randomized GPU parity sweeps: 120 configurations drawn once from a
fixed seed across the entry points (decode, prefill, atlas_attend_mods), the
dtype pairs (fp32, bf16, fp32 queries over a bf16 cache), head dims, page
sizes, GQA ratios, ragged context lengths, per-sequence window / sink /
softcap settings and the modifications (non-causal rows, ALiBi slopes, mask
bits), each run through the C ABI on NaN-poisoned arenas and checked
against the fp64 oracle at the dtype's bar; and 40 decodes over regenerated
K/V (cold pages regenerated into scratch, or generated inside the fold)
with random resident shares, sequence keys, layers and variants, against
the oracle's own generator.  Each case prints itself first (its id names
every drawn parameter)."""
import math

import numpy as np
import pytest
import torch

import harness as H
import workloads
from test_gpu_mods import alibi_slopes, check_mods, make_mask, run_mods

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_paged_causal_amd  # noqa: F401  (fails loudly if libatlas.so is missing)
    yield


def say(*a):
    print(*a, flush=True)


def draw_cases(seed=20261203, n=120):
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        kind = str(rng.choice(["decode", "prefill", "mods"], p=[0.4, 0.35, 0.25]))
        pair = str(rng.choice(["f32", "bf16", "f32q"]))
        d = int(rng.choice([64, 128]))
        page = int(rng.choice([1, 2, 16, 64, 512]))
        hkv = int(rng.choice([1, 2, 4]))
        group = int(rng.choice([1, 2, 4, 8]))
        batch = int(rng.integers(1, 4))
        q_len = 1 if kind == "decode" else int(rng.choice([2, 17, 64, 100, 257]))
        lens = tuple(int(x) for x in rng.integers(q_len, q_len + 1500, size=batch))
        c = dict(k=k, kind=kind, pair=pair, d=d, page=page, hkv=hkv, hq=hkv * group, q_len=q_len, lens=lens,
                 window=None, sinks=None, softcap=None, causal=True, alibi=False, density=None)
        if kind != "mods" and rng.random() < 0.5:
            c["window"] = tuple(int(x) for x in rng.choice([0, 16, 100, 700], size=batch))
            c["sinks"] = tuple(int(x) for x in rng.integers(0, 5, size=batch))
            c["softcap"] = tuple(float(x) for x in rng.choice([0.0, 2.0, 30.0], size=batch))
        if kind == "mods":
            c["causal"] = bool(rng.random() < 0.6)
            c["alibi"] = bool(rng.random() < 0.6)
            c["density"] = [None, 0.3, 0.9][int(rng.integers(0, 3))]
            if not c["alibi"] and c["density"] is None and c["causal"]:
                c["causal"] = False      # keep every mods case a real modification
        cases.append(c)
    return cases


CASES = draw_cases()


def case_id(c):
    s = f"{c['k']}-{c['kind']}-{c['pair']}-d{c['d']}-p{c['page']}-h{c['hq']}x{c['hkv']}-q{c['q_len']}-L{max(c['lens'])}"
    if c["window"] is not None:
        s += "-var"
    if c["kind"] == "mods":
        s += f"-{'c' if c['causal'] else 'nc'}{'-alibi' if c['alibi'] else ''}{'-mask' if c['density'] else ''}"
    return s


def workload_of(c):
    dtype = "f32" if c["pair"] == "f32" else "bf16"
    w = workloads.Workload(f"sweep{c['k']}", seed=300 + c["k"], batch=len(c["lens"]), hq=c["hq"], hkv=c["hkv"],
                           head_dim=c["d"], page_size=c["page"], dtype=dtype, q_len=c["q_len"],
                           context_lens=np.asarray(c["lens"], np.int32), scale=1.0 / math.sqrt(c["d"]),
                           shuffle_pages=True, q_dtype="f32" if c["pair"] == "f32q" else None)
    if c["window"] is not None:
        w.window = np.asarray(c["window"], np.int32)
        w.sinks = np.asarray(c["sinks"], np.int32)
        w.softcap = np.asarray(c["softcap"], np.float32)
    return w


@pytest.mark.parametrize("c", CASES, ids=case_id)
def test_sweep_matches_oracle(c):
    say(f"[sweep] {case_id(c)} lens={c['lens']} window={c['window']} sinks={c['sinks']} softcap={c['softcap']}")
    w = workload_of(c)
    inp = H.build(w, poison=True, extra_phys=2)
    if c["kind"] == "mods":
        slopes = alibi_slopes(w.hq) if c["alibi"] else None
        mask = make_mask(w, c["density"], seed=900 + c["k"]) if c["density"] else None
        out, lse = run_mods(inp, c["causal"], slopes, mask)
        torch.cuda.synchronize()
        check_mods(inp, out, lse, c["causal"], slopes, mask, case_id(c))
    else:
        out, lse = H.run(inp, entry=c["kind"])
        torch.cuda.synchronize()
        H.check_against_oracle(inp, out, lse, what=case_id(c))


def draw_regen_cases(seed=20261204, n=40):
    """Decodes over regenerated K/V: cold pages regenerated into scratch and
    then read ("scratch"), or generated inside the fold ("fused"), with a
    random resident share, sequence keys and variants."""
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        batch = int(rng.integers(1, 4))
        hkv = int(rng.choice([1, 2, 4]))
        c = dict(k=k, mode=str(rng.choice(["scratch", "fused"])), dtype=str(rng.choice(["f32", "bf16", "f32q"])),
                 d=int(rng.choice([64, 128])), page=int(rng.choice([1, 16, 64, 512])), hkv=hkv,
                 hq=hkv * int(rng.choice([1, 2, 4, 8])), hot=float(rng.choice([0.0, 0.25, 0.6, 1.0])),
                 lens=tuple(int(x) for x in rng.integers(1, 2000, size=batch)),
                 keys=tuple(int(x) for x in rng.choice(65536, size=batch, replace=False)) if rng.random() < 0.5
                 else None, window=None, sinks=None, softcap=None, layer=int(rng.integers(0, 40)))
        if rng.random() < 0.4:
            c["window"] = tuple(int(x) for x in rng.choice([0, 16, 300], size=batch))
            c["sinks"] = tuple(int(x) for x in rng.integers(0, 4, size=batch))
            c["softcap"] = tuple(float(x) for x in rng.choice([0.0, 5.0], size=batch))
        cases.append(c)
    return cases


REGEN_CASES = draw_regen_cases()


def regen_id(c):
    s = (f"{c['k']}-{c['mode']}-{c['dtype']}-d{c['d']}-p{c['page']}-h{c['hq']}x{c['hkv']}-hot{c['hot']}"
         f"-L{max(c['lens'])}")
    return s + ("-keys" if c["keys"] else "") + ("-var" if c["window"] else "")


@pytest.mark.parametrize("c", REGEN_CASES, ids=regen_id)
def test_sweep_regenerated_decode_matches_oracle(c):
    import exact_paged_causal_amd as atlas
    say(f"[sweep-regen] {regen_id(c)} lens={c['lens']} keys={c['keys']} window={c['window']} layer={c['layer']}")
    dtype = "f32" if c["dtype"] == "f32" else "bf16"
    w = workloads.Workload(f"sweepregen{c['k']}", seed=500 + c["k"], batch=len(c["lens"]), hq=c["hq"],
                           hkv=c["hkv"], head_dim=c["d"], page_size=c["page"], dtype=dtype, q_len=1,
                           context_lens=np.asarray(c["lens"], np.int32), scale=1.0 / math.sqrt(c["d"]),
                           regenerated=True, hot_fraction=c["hot"], shuffle_pages=True,
                           q_dtype="f32" if c["dtype"] == "f32q" else None,
                           seq_keys=None if c["keys"] is None else np.asarray(c["keys"], np.int32))
    w.layer = c["layer"]
    if c["window"] is not None:
        w.window = np.asarray(c["window"], np.int32)
        w.sinks = np.asarray(c["sinks"], np.int32)
        w.softcap = np.asarray(c["softcap"], np.float32)
    inp = H.build(w)
    if c["mode"] == "scratch":
        out, lse = H.run(inp)
    else:
        pt = inp.layout.page_table.copy()
        for seq, lp, _ in inp.layout.cold_jobs:
            pt[seq, lp] = atlas.ATLAS_PAGE_REGENERATE
        out, lse = atlas.atlas_attend_decode_regen(inp.q, inp.k, inp.v, torch.from_numpy(pt).cuda(),
                                                   inp.context_lens, w.scale, seed=w.seed, layer=w.layer,
                                                   seq_keys=H.seq_keys_tensor(w), window=inp.window,
                                                   sink_tokens=inp.sinks, softcap=inp.softcap)
    torch.cuda.synchronize()
    H.check_against_oracle(inp, out, lse, what=regen_id(c))

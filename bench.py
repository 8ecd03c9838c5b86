"""Benchmark of the paged-attention hot path on one MI355X.

One step = one pass of the whole hot path over the synthetic inputs:
  * long-context paged decode (B=8 x 65536 tokens, Hq=32, Hkv=8, D=64,
    pages of 512, fp32, 25 % of pages resident): the cold 75 % of pages are
    regenerated into scratch on the device, then the split-KV fold and the
    log-sum-exp merge run over resident + scratch pages;
  * causal GQA prefill (S=8192, Hq=32, Hkv=8, D=128, bf16, pages of 128 in a
    random physical order) on the tiled matrix-core kernel.
Inputs are resident in HBM before timing starts.  `value` is the decode
attention pass's K/V-read throughput (algorithmic bytes / time of the
attention call, split + merge); the prefill throughput and the regenerator
are reported beside it.  Per-kernel times are medians over the timed steps
of HIP events recorded on the stream the kernels run on (--step-times prints
every step's).  After the timed steps, the three smaller
synthetic workloads (single-head decode, GQA short-query suffix attention,
mixed-length decode with window / sinks / softcap) are timed per call and
reported under "workloads" with the two step workloads, and the long-context
decode is run once more with its cold pages generated inside the attention
kernel (atlas_attend_decode_regen) instead of regenerated into scratch
("next": "fused_regen_decode"; its output is compared bit for bit with the
step's); the K/V append of a decode step and of a whole prefill history is
timed under "next": "append_kv", the prefill shape with a window, sinks
and a softcap under "next": "prefill_variants", and the same shape with
fp32 Q/K/V (split fp16 operands on the matrix cores, plain and with
ALiBi or a document mask) under "next": "prefill_f32", and atlas_attend_mods on the same bf16 shape (ALiBi
causal and non-causal, a block-diagonal document mask) under "next": "mods";
the long-context decode through the hot-page cache (atlas_cache_plan ->
regenerate admitted pages -> decode with the rest generated in the kernel)
under "next": "hot_cache"; short prefill chunks behind a 32768-token history
(the tiled kernels with key splits) under "next": "chunked_prefill";
single-sequence decodes over 131072 keys (many splits per row) and single
queries from 128 q-heads per K/V head (decode and prefill entries) under
"next": "few_item".
A plain 256 MiB device-to-device copy is timed last as context for the HBM
figures ("hbm_context"); the small workloads also report one C-ABI call
with prepared arguments ("c_abi_us") beside the Python-call time.
"provenance" names the GPU, its shader clock as rocm-smi reads it right
after the timed steps, the host CPU model and thread count, the ROCm, HIP and
torch versions and the git commit.  The fp64 CPU oracle is timed on the
host's cores as a baseline (not a target): on the whole decode workload in
GB/s ("cpu_baseline") and on a bounded sample of the prefill in GFLOP/s
("prefill": "cpu_baseline"), each also checking the GPU output it covers.

Prints one JSON line.  `--gpus N` with N > 1 exits: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Sources of each profiled kernel: the HBM traffic measured with rocprofv3
# counters (profiles/traffic.json) is reported only while these files still
# hash to what was profiled; otherwise `traffic` is null.
PROFILED_SOURCES = {
    "decode_split_long_context": ["split_valu.hip", "merge.hip", "merge_row.h", "philox.h", "plan.h", "device.h",
                                  "kernels.h"],
    "prefill_tiled_causal_8192": ["prefill_mfma.hip", "device.h", "kernels.h"],
    "regen_long_context": ["regen.hip", "philox.h", "device.h", "kernels.h"],
}

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak, TFLOP/s
METRIC = "decode attn KV-read GB/s (% HBM peak); prefill TFLOP/s (% MFMA peak)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--step-times", action="store_true",
                    help="print every timed step's kernel durations (us) to stderr")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the per-call timing of the three smaller workloads")
    ap.add_argument("--workloads-only", action="store_true",
                    help="diagnostic: time only the three smaller workloads (for a kernel trace of them)")
    ap.add_argument("--report-warmup", type=int, default=5,
                    help="warm-up calls before each report's timed calls (at least)")
    ap.add_argument("--report-warmup-s", type=float, default=0.1,
                    help="warm-up seconds before each report's timed calls (at least; 0: count only)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="kept for the recorded profiling commands: the plain 256 MiB device copy "
                         "(HBM counter calibration and context) now always runs")
    return ap.parse_args()


def measured_traffic(key):
    """Calibrated HBM bytes per call (fetch + write) from profiles/traffic.json,
    or None when the kernel's sources changed since the counters were taken."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))[key]
    except (OSError, KeyError, ValueError):
        return None
    h = hashlib.sha256()
    for f in PROFILED_SOURCES[key]:
        h.update(open(os.path.join(ROOT, "exact_paged_causal_amd", "csrc", f), "rb").read())
    if h.hexdigest()[:16] != rec.get("sources_sha"):
        return None
    return int(round(rec["fetch_bytes"] + rec["write_bytes"]))


class Timer:
    """HIP-event timing of one launch sequence on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def __call__(self, fn):
        t = self.torch
        s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        s.record()
        r = fn()
        e.record()
        self.pairs.append((s, e))
        return r

    def ms(self):
        return [s.elapsed_time(e) for s, e in self.pairs]


def decode_setup(torch, workloads, atlas):
    w = workloads.make("long_context_decode")
    lay = workloads.page_layout(w)
    shape = workloads.arena_shape(w, lay.num_phys)
    k = torch.zeros(shape, dtype=torch.float32, device="cuda")
    v = torch.zeros_like(k)
    hot = torch.from_numpy(lay.hot_jobs).cuda()
    cold = torch.from_numpy(lay.cold_jobs).cuda()
    atlas.atlas_regenerate_pages(k, v, hot, seed=w.seed, layer=w.layer)
    q = workloads.randn(workloads.query_shape(w), seed=w.seed * 100 + 1, device="cuda")
    pt = torch.from_numpy(lay.page_table).cuda()
    ctx = torch.from_numpy(w.context_lens).cuda()
    return dict(w=w, lay=lay, k=k, v=v, hot=hot, cold=cold, q=q, pt=pt, ctx=ctx)


def prefill_setup(torch, workloads, np):
    w = workloads.make("causal_prefill")
    lay = workloads.page_layout(w)
    shape = workloads.arena_shape(w, lay.num_phys)
    n = lay.num_phys
    kl = workloads.randn(shape, seed=w.seed * 100 + 2, dtype="bf16", device="cuda")
    vl = workloads.randn(shape, seed=w.seed * 100 + 3, dtype="bf16", device="cuda")
    ids = torch.from_numpy(lay.page_table[0, :n].astype(np.int64)).cuda()
    k = torch.empty_like(kl)
    v = torch.empty_like(vl)
    k.index_copy_(0, ids, kl)
    v.index_copy_(0, ids, vl)
    q = workloads.randn(workloads.query_shape(w), seed=w.seed * 100 + 1, dtype="bf16", device="cuda")
    pt = torch.from_numpy(lay.page_table).cuda()
    ctx = torch.from_numpy(w.context_lens).cuda()
    return dict(w=w, lay=lay, k=k, v=v, q=q, pt=pt, ctx=ctx, kl=kl, vl=vl)


# Warm-up before each report's timed calls: at least REPORT_WARMUP[0] calls
# and REPORT_WARMUP[1] seconds of them (--report-warmup, --report-warmup-s).
REPORT_WARMUP = [5, 0.1]


def _median_call_us(torch, np, fn, calls=30, warm=None, warm_s=None):
    """Median HIP-event time of `calls` back-to-back calls, after at least
    `warm` calls and `warm_s` seconds of them (the clocks ramp back up after
    host-only set-up phases)."""
    warm = REPORT_WARMUP[0] if warm is None else warm
    warm_s = REPORT_WARMUP[1] if warm_s is None else warm_s
    t0 = time.perf_counter()
    n = 0
    while n < warm or time.perf_counter() - t0 < warm_s:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t = Timer(torch)
    for _ in range(calls):
        t(fn)
    torch.cuda.synchronize()
    return float(np.median(t.ms())) * 1000.0


def _call_stats_us(torch, np, fn, calls=50):
    """(median, min) HIP-event time in us of `calls` back-to-back calls after
    the report warm-up."""
    warm, warm_s = REPORT_WARMUP
    t0 = time.perf_counter()
    n = 0
    while n < warm or time.perf_counter() - t0 < warm_s:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t = Timer(torch)
    for _ in range(calls):
        t(fn)
    torch.cuda.synchronize()
    ms = np.array(t.ms())
    return float(np.median(ms)) * 1000.0, float(ms.min()) * 1000.0


def _oracle_timed(run, min_seconds):
    """Call run() until at least min_seconds of timed work; returns (calls, seconds)."""
    n, secs = 0, 0.0
    while secs < min_seconds or n == 0:
        t0 = time.perf_counter()
        run()
        secs += time.perf_counter() - t0
        n += 1
    return n, secs


def _c_abi_call_us(torch, np, entry, args, calls=30):
    """Median time of one C-ABI call with prepared arguments (outputs and
    workspace already set): what a native caller pays per call, without the
    Python binding's argument marshalling."""
    import ctypes
    from exact_paged_causal_amd.atlas import lib
    fn = getattr(lib, entry)
    sh = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ref = ctypes.byref(args)

    def call():
        st = fn(ref, sh)
        if st != 0:
            raise RuntimeError(f"{entry} returned {st}")
    return _median_call_us(torch, np, call, calls=calls)


def _graph10_us(torch, np, prep):
    """Time per call of a HIP graph holding ten copies of a prepared call
    (as a model step's layers would be captured), captured on a side stream
    after an eager call there."""
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        prep()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for _ in range(10):
            prep()
    torch.cuda.synchronize()
    us = _median_call_us(torch, np, g.replay, calls=50) / 10
    del g
    return us


def _arena(torch, workloads, np, w, lay):
    """Device K/V arenas of a non-regenerated workload: seeded logical pages
    scattered to their physical ids."""
    kl, vl, n_pages = workloads.logical_kv(w, "cuda")
    shape = workloads.arena_shape(w, lay.num_phys)
    k = torch.zeros(shape, dtype=kl.dtype, device="cuda")
    v = torch.zeros_like(k)
    ids = torch.from_numpy(np.concatenate([lay.page_table[b, :n_pages[b]]
                                           for b in range(w.batch)]).astype(np.int64)).cuda()
    k.index_copy_(0, ids, kl)
    v.index_copy_(0, ids, vl)
    return k, v


def fused_report(torch, np, d, atlas, dec_ms, regen_ms, calls=30):
    """Long-context decode with the cold pages generated inside the fold
    (atlas_attend_decode_regen) instead of regenerated into scratch: same
    inputs and outputs as one regenerate + decode step, compared bit for bit
    with the step's own output."""
    w, lay = d["w"], d["lay"]
    pt = lay.page_table.copy()
    for seq, lp, _ in lay.cold_jobs:
        pt[seq, lp] = -1
    pt = torch.from_numpy(pt).cuda()
    out = torch.empty(w.batch, 1, w.hq, w.head_dim, dtype=torch.float32, device="cuda")
    ref = torch.empty_like(out)
    atlas.atlas_regenerate_pages(d["k"], d["v"], d["cold"], seed=w.seed, layer=w.layer)
    atlas.atlas_attend_decode(d["q"], d["k"], d["v"], d["pt"], d["ctx"], w.scale, out=ref)
    call = lambda: atlas.atlas_attend_decode_regen(d["q"], d["k"], d["v"], pt, d["ctx"], w.scale,
                                                   seed=w.seed, layer=w.layer, out=out)
    us = _median_call_us(torch, np, call, calls=calls)
    torch.cuda.synchronize()
    n_cold, n_pages = int(lay.cold_jobs.shape[0]), int(lay.page_table.size)
    per_page = w.hkv * w.page_size * w.head_dim * 4 * 2
    unfused = (dec_ms + regen_ms) * 1000.0
    return {"us": round(us, 1), "unfused_us": round(unfused, 1), "speedup": round(unfused / us, 3),
            "hot_kv_bytes_read": (n_pages - n_cold) * per_page, "cold_kv_bytes_generated": n_cold * per_page,
            "generated_values": n_cold * per_page // 4,
            "bitwise_equal_to_unfused": bool(torch.equal(out, ref)),
            "note": "atlas_attend_decode_regen: cold pages (page-table -1) generated in the fold's registers"}


def prefill_variants_report(torch, np, p, atlas, calls=10):
    """The causal-prefill shape (S=8192, Hq=32, Hkv=8, D=128, bf16) with the
    mixed-decode workload's variants on the tiled kernel: window 4096, 4 sink
    keys, softcap 50.  Throughput counts the visible (query, key) pairs only:
    key blocks before a query block's window are skipped."""
    pw = p["w"]
    S, hq, d = pw.q_len, pw.hq, pw.head_dim
    W, n_s, capv = 4096, 4, 50.0
    win = torch.full((1,), W, dtype=torch.int32, device="cuda")
    snk = torch.full((1,), n_s, dtype=torch.int32, device="cuda")
    cap = torch.full((1,), capv, dtype=torch.float32, device="cuda")
    out = torch.empty(1, S, hq, d, dtype=torch.float32, device="cuda")
    call = lambda: atlas.atlas_attend_prefill(p["q"], p["k"], p["v"], p["pt"], p["ctx"], pw.scale, window=win,
                                              sink_tokens=snk, softcap=cap, out=out)
    us = _median_call_us(torch, np, call, calls=calls)
    pos = np.arange(S, dtype=np.int64)
    vis = np.minimum(pos + 1, W) + np.minimum(n_s, np.maximum(pos + 1 - W, 0))
    flops = 4.0 * d * hq * float(vis.sum())
    return {"us": round(us, 1), "flop": flops, "TFLOPs": round(flops / us / 1e6, 1),
            "frac_mfma": round(flops / us / 1e6 / BF16_PEAK_TFLOPS, 4),
            "note": "window 4096 + 4 sinks + softcap 50 on the causal-prefill shape; visible pairs only"}


def _document_mask(torch, np, S, words, doc=2048):
    """Packed causal block-diagonal mask of S query rows over words * 32 keys:
    documents of `doc` tokens, query i at position i."""
    j = np.arange(words * 32)
    qpos = np.arange(S)
    keep = (j[None, :] // doc == qpos[:, None] // doc) & (j[None, :] <= qpos[:, None])
    bits = np.packbits(keep, axis=-1, bitorder="little").view("<u4").astype(np.uint32).view(np.int32)
    return torch.from_numpy(np.ascontiguousarray(bits)[None]).cuda()


def prefill_f32_report(torch, np, workloads, atlas, calls=10):
    """The causal-prefill shape (S=8192, Hq=32, Hkv=8, D=128, pages of 128)
    with fp32 Q/K/V: the tiled kernel on split fp16 operands.  TFLOP/s counts
    the method's 4 D flop per (q-head, visible pair); each of its products
    issues three fp16 matrix products, so the matrix cores run 3x that.  The
    same shape through atlas_attend_mods: ALiBi on causal rows, and four
    2048-token documents under a causal block-diagonal mask."""
    w = workloads.make("causal_prefill", dtype="f32")
    lay = workloads.page_layout(w)
    k, v = _arena(torch, workloads, np, w, lay)
    q = workloads.randn(workloads.query_shape(w), seed=w.seed * 100 + 1, dtype="f32", device="cuda")
    pt = torch.from_numpy(lay.page_table).cuda()
    ctx = torch.from_numpy(w.context_lens).cuda()
    out = torch.empty(workloads.query_shape(w), dtype=torch.float32, device="cuda")
    lse = torch.empty(w.batch, w.q_len, w.hq, dtype=torch.float32, device="cuda")
    call = lambda: atlas.atlas_attend_prefill(q, k, v, pt, ctx, w.scale, out=out, lse=lse)
    us = _median_call_us(torch, np, call, calls=calls)
    S = w.q_len
    flops = 4.0 * w.head_dim * w.hq * S * (S + 1) / 2
    tf = flops / us / 1e6
    slopes = torch.tensor(2.0 ** (-8.0 * (np.arange(w.hq) + 1) / w.hq), dtype=torch.float32, device="cuda")
    doc = 2048
    mask = _document_mask(torch, np, S, (int(pt.shape[1]) * w.page_size + 31) // 32, doc)
    mods = {}
    for name, kw, pairs in (("alibi_causal", dict(alibi_slopes=slopes), S * (S + 1) / 2),
                            ("document_mask", dict(mask_bits=mask), (S // doc) * doc * (doc + 1) / 2)):
        mcall = lambda: atlas.atlas_attend_mods(q, k, v, pt, ctx, w.scale, out=out, lse=lse, **kw)
        mus = _median_call_us(torch, np, mcall, calls=calls)
        fl = 4.0 * w.head_dim * w.hq * pairs
        mods[name] = {"us": round(mus, 1), "flop": fl, "TFLOPs": round(fl / mus / 1e6, 1)}
    return {"us": round(us, 1), "flop": flops, "TFLOPs": round(tf, 1),
            "frac_mfma_fp16": round(3.0 * tf / BF16_PEAK_TFLOPS, 4), "mods": mods,
            "note": "fp32 Q/K/V; every product as three fp16 matrix products (hi.hi + lo.hi + hi.lo); "
                    "mods TFLOP/s over visible pairs"}


def mods_report(torch, np, p, atlas, calls=10):
    """atlas_attend_mods on the causal-prefill shape (S=8192, Hq=32, Hkv=8,
    D=128, bf16): ALiBi slopes 2^(-8(h+1)/Hq) on causal and on non-causal rows,
    and a causal block-diagonal mask of four 2048-token documents (packed
    sequences).  TFLOP/s counts the visible pairs; the tiled kernel drops the
    key blocks a mask hides from every row of a query block and applies the
    mask per element inside the others."""
    pw = p["w"]
    S, hq, d = pw.q_len, pw.hq, pw.head_dim
    slopes = torch.tensor(2.0 ** (-8.0 * (np.arange(hq) + 1) / hq), dtype=torch.float32, device="cuda")
    doc = 2048
    mask = _document_mask(torch, np, S, (int(p["pt"].shape[1]) * pw.page_size + 31) // 32, doc)
    out = torch.empty(1, S, hq, d, dtype=torch.float32, device="cuda")
    lse = torch.empty(1, S, hq, dtype=torch.float32, device="cuda")
    rep = {}
    for name, kw, pairs in (("alibi_causal", dict(alibi_slopes=slopes), S * (S + 1) / 2),
                            ("alibi_noncausal", dict(alibi_slopes=slopes, causal=False), float(S) * S),
                            ("document_mask", dict(mask_bits=mask), (S // doc) * doc * (doc + 1) / 2)):
        call = lambda: atlas.atlas_attend_mods(p["q"], p["k"], p["v"], p["pt"], p["ctx"], pw.scale, out=out,
                                               lse=lse, **kw)
        us = _median_call_us(torch, np, call, calls=calls)
        fl = 4.0 * d * hq * pairs
        rep[name] = {"us": round(us, 1), "flop": fl, "TFLOPs": round(fl / us / 1e6, 1)}
    rep["note"] = "bf16 tiled kernel; TFLOP/s over visible pairs; key blocks a mask hides entirely are skipped"
    return rep


def cache_report(torch, np, workloads, atlas, calls=10):
    """The long-context decode (B=8 x 65536 tokens, Hkv=8, D=64, fp32, pages
    of 512 = 2 MiB of K/V each) through the hot-page cache with the CFR-Atlas
    example's policy (256 MiB budget, KeepRecent 2048 tokens, admit
    regenerated pages) and with a 2 GiB budget that holds every page.  One
    call = host plan + regeneration of the admitted pages + decode with the
    other pages generated in the kernel; first call and steady state."""
    w = workloads.make("long_context_decode")
    B, P, maxp = w.batch, w.page_size, int(w.context_lens.max()) // w.page_size
    page_bytes = w.hkv * P * w.head_dim * 4 * 2
    q = workloads.randn(workloads.query_shape(w), seed=w.seed * 100 + 1, device="cuda")
    ctx = torch.from_numpy(w.context_lens).cuda()
    lens = w.context_lens.astype(np.int32)
    seq_ids = list(range(B))                # each sequence's id is its generator key
    keys = torch.tensor(seq_ids, dtype=torch.int32, device="cuda")
    rep = {}
    for name, budget in (("budget_256MiB", 256 << 20), ("budget_2GiB", 2 << 30)):
        cache = atlas.HotCache(budget, page_bytes, P, recent_tokens=2048, admit_regenerated=True)
        cap = max(budget // page_bytes, 1)
        k = torch.zeros((cap, w.hkv, P, w.head_dim), device="cuda")
        v = torch.zeros_like(k)
        plan_us = []
        # The plan's page table goes up through a pinned staging buffer with
        # an asynchronous copy (a pageable copy would block the host); each
        # call below ends with a device synchronisation before the buffer is
        # written again.
        pt_pin = torch.empty((B, maxp), dtype=torch.int32).pin_memory()
        pt_dev = torch.empty((B, maxp), dtype=torch.int32, device="cuda")

        def call():
            t0 = time.perf_counter()
            pt, jobs = cache.plan(w.layer, seq_ids, lens, maxp)
            plan_us.append((time.perf_counter() - t0) * 1e6)
            if len(jobs):
                atlas.atlas_regenerate_pages(k, v, torch.from_numpy(jobs).cuda(), seed=w.seed, layer=w.layer)
            pt_pin.numpy()[:] = pt
            pt_dev.copy_(pt_pin, non_blocking=True)
            if cache.last_cold:
                atlas.atlas_attend_decode_regen(q, k, v, pt_dev, ctx, w.scale, seed=w.seed,
                                                layer=w.layer, seq_keys=keys)
            else:   # every page resident: the plain decode, same bits
                atlas.atlas_attend_decode(q, k, v, pt_dev, ctx, w.scale)

        torch.cuda.synchronize()
        t0 = time.perf_counter()
        call()
        torch.cuda.synchronize()
        first_us = (time.perf_counter() - t0) * 1e6
        walls = []
        for _ in range(calls):
            t0 = time.perf_counter()
            call()
            torch.cuda.synchronize()
            walls.append((time.perf_counter() - t0) * 1e6)
        st = cache.stats()
        # The same decode call on the same arenas and page table, without the
        # plan and the upload, timed the same way (wall clock with a device
        # synchronisation).
        plain = []
        for _ in range(calls if not cache.last_cold else 0):
            t0 = time.perf_counter()
            atlas.atlas_attend_decode(q, k, v, pt_dev, ctx, w.scale)
            torch.cuda.synchronize()
            plain.append((time.perf_counter() - t0) * 1e6)
        rep[name] = {"first_call_us": round(first_us, 1), "steady_call_us": round(float(np.median(walls)), 1),
                     "plan_us": round(float(np.median(plan_us[1:])), 1), "resident_pages": st["resident_pages"],
                     "cold_pages_per_call": int(cache.last_cold),
                     "entry": "atlas_attend_decode_regen" if cache.last_cold else "atlas_attend_decode",
                     "resident_bytes": st["resident_bytes"]}
        if not cache.last_cold:
            rep[name]["plain_decode_call_us"] = round(float(np.median(plain)), 1)
        cache.close()
        del k, v
    rep["note"] = ("wall time per call with a device synchronisation (host plan and page-table upload included); "
                   "cold pages are generated inside the decode kernel, so no scratch memory is used; a plan that "
                   "leaves no page cold runs the plain decode (same bits); plain_decode_call_us: that decode alone, "
                   "timed the same way")
    return rep


def chunked_prefill_report(torch, np, workloads, atlas, calls=10):
    """Prefill chunks of 128 and 512 queries behind a 32768-token history
    (B=1, Hq=32, Hkv=8, D=128, pages of 128), bf16 and fp32: few query blocks,
    so the tiled kernels split each block's keys across workgroups and the
    LSE merge combines them.  TFLOP/s over the visible pairs."""
    rep = {}
    for dtype, q_len in (("bf16", 128), ("bf16", 512), ("f32", 512)):
        L = 32768
        w = workloads.make("causal_prefill", dtype=dtype, q_len=q_len, context_lens=np.array([L], np.int32))
        lay = workloads.page_layout(w)
        k, v = _arena(torch, workloads, np, w, lay)
        q = workloads.randn(workloads.query_shape(w), seed=3, dtype=dtype, device="cuda")
        pt = torch.from_numpy(lay.page_table).cuda()
        ctx = torch.from_numpy(w.context_lens).cuda()
        args, _ = atlas.make_attn_args(q, k, v, pt, ctx, w.scale)
        ws = torch.empty(atlas.atlas_prefill_workspace_bytes(args), dtype=torch.uint8, device="cuda")
        out = torch.empty(workloads.query_shape(w), dtype=torch.float32, device="cuda")
        lse = torch.empty(1, q_len, w.hq, dtype=torch.float32, device="cuda")
        call = lambda: atlas.atlas_attend_prefill(q, k, v, pt, ctx, w.scale, out=out, lse=lse, workspace=ws)
        us = _median_call_us(torch, np, call, calls=calls)
        fl = 4.0 * w.head_dim * w.hq * (q_len * L - q_len * (q_len - 1) / 2)
        rep[f"{dtype}_q{q_len}_L{L}"] = {"us": round(us, 1), "flop": fl, "TFLOPs": round(fl / us / 1e6, 1)}
        del k, v
    rep["note"] = "tiled prefill with key splits + LSE merge (workgroups per query block x splits)"
    return rep


def few_item_report(torch, np, workloads, atlas, calls=10):
    """Calls with few (sequence, K/V head) work items over long contexts
    (D=128, pages of 128): single-sequence decodes over 131072 keys, which
    the split plan spreads over up to 512 splits per row (merged by eight
    waves per row past 64), and 8 single queries from 128 q-heads over one
    K/V head at 32768 keys through the decode entry (split-KV folds) and
    the prefill entry (tiled kernels).  GB/s of visible K/V."""
    rep = {}
    for name, dtype, entry, B, hq, hkv, L in (("decode_f32_h8x1_B1_L131072", "f32", "decode", 1, 8, 1, 131072),
                                             ("decode_bf16_h32x8_B1_L131072", "bf16", "decode", 1, 32, 8, 131072),
                                             ("decode_bf16_h64x1_B1_L131072", "bf16", "decode", 1, 64, 1, 131072),
                                             ("decode_bf16_h128x1_B8_L32768", "bf16", "decode", 8, 128, 1, 32768),
                                             ("prefill_q1_bf16_h128x1_B8_L32768", "bf16", "prefill", 8, 128, 1,
                                              32768)):
        w = workloads.make("causal_prefill", dtype=dtype, q_len=1, batch=B, hq=hq, hkv=hkv,
                           context_lens=np.full(B, L, np.int32))
        lay = workloads.page_layout(w)
        k, v = _arena(torch, workloads, np, w, lay)
        q = workloads.randn(workloads.query_shape(w), seed=3, dtype=dtype, device="cuda")
        pt = torch.from_numpy(lay.page_table).cuda()
        ctx = torch.from_numpy(w.context_lens).cuda()
        args, _ = atlas.make_attn_args(q, k, v, pt, ctx, w.scale)
        wsb = atlas.atlas_decode_workspace_bytes(args) if entry == "decode" else atlas.atlas_prefill_workspace_bytes(args)
        ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
        out = torch.empty(workloads.query_shape(w), dtype=torch.float32, device="cuda")
        lse = torch.empty(B, 1, hq, dtype=torch.float32, device="cuda")
        fn = atlas.atlas_attend_decode if entry == "decode" else atlas.atlas_attend_prefill
        call = lambda: fn(q, k, v, pt, ctx, w.scale, out=out, lse=lse, workspace=ws)
        us = _median_call_us(torch, np, call, calls=calls)
        kv_bytes = 2.0 * B * L * hkv * w.head_dim * (4 if dtype == "f32" else 2)
        rep[name] = {"us": round(us, 1), "GBps": round(kv_bytes / us / 1e3, 1)}
        del k, v
    rep["note"] = "few work items per split: plan of up to 512 splits per row; one query, 128 q-heads per K/V head"
    return rep


def append_report(torch, np, workloads, atlas):
    """K/V append: the long-context decode step's write of one new token per
    sequence (B=8, Hkv=8, D=64, fp32, into pages of 512), and a bulk append of
    a whole 8192-token bf16 history (Hkv=8, D=128, pages of 128) -- a copy
    bound by HBM (each byte read once and written once)."""
    rep = {}
    for name, B, n_new, hkv, d, P, dtype in (("decode_step", 8, 1, 8, 64, 512, "f32"),
                                             ("bulk_8192", 1, 8192, 8, 128, 128, "bf16")):
        maxp = (65536 + P - 1) // P if name == "decode_step" else 8192 // P
        phys = B * maxp
        k = torch.zeros((phys, hkv, P, d), dtype=torch.float32 if dtype == "f32" else torch.bfloat16,
                        device="cuda")
        v = torch.zeros_like(k)
        kn = workloads.randn((B, n_new, hkv, d), seed=5, dtype=dtype, device="cuda")
        vn = workloads.randn((B, n_new, hkv, d), seed=6, dtype=dtype, device="cuda")
        pt = torch.from_numpy(np.random.default_rng(9).permutation(phys).astype(np.int32).reshape(B, maxp)).cuda()
        start = torch.full((B,), 65535 if name == "decode_step" else 0, dtype=torch.int32, device="cuda")
        us = _median_call_us(torch, np, lambda: atlas.atlas_append_kv(k, v, kn, vn, pt, start))
        nbytes = 2 * kn.numel() * kn.element_size()
        rep[name] = {"us": round(us, 2), "bytes_written": nbytes,
                     "GBs_read_plus_written": round(2 * nbytes / us / 1e3, 1)}
        del k, v
    rep["note"] = ("decode_step is launch-latency bound (32 KiB); bulk_8192 moves 32 MiB of K/V "
                   "(read + write counted)")
    torch.cuda.empty_cache()
    return rep


def workload_report(torch, np, workloads, atlas, oracle=None):
    """The three smaller synthetic workloads, each timed per call (median and
    minimum of 50 after the report warm-up): single-head decode (all pages
    resident, and all 8 pages regenerated inside the call), the GQA
    short-query suffix attention, and the mixed-length decode with window /
    sinks / softcap on even sequences.  With the oracle module given, each
    also gets a cpu_baseline: the oracle timed on the same inputs (the whole
    workload, or a stated sample) in the workload's unit, checking the GPU
    output it covers."""
    rep = {}
    # Single-head decode: 2 MiB of K/V, launch-latency bound.
    w = workloads.make("single_head_decode")
    for mode, hf in (("resident", 1.0), ("cold", 0.0)):
        lay = workloads.page_layout(w, hot_fraction=hf)
        shape = workloads.arena_shape(w, lay.num_phys)
        k = torch.zeros(shape, dtype=torch.float32, device="cuda")
        v = torch.zeros_like(k)
        if len(lay.hot_jobs):
            atlas.atlas_regenerate_pages(k, v, torch.from_numpy(lay.hot_jobs).cuda(), seed=w.seed, layer=w.layer)
        cold = torch.from_numpy(lay.cold_jobs).cuda() if len(lay.cold_jobs) else None
        q = workloads.randn(workloads.query_shape(w), seed=w.seed * 100 + 1, device="cuda")
        pt = torch.from_numpy(lay.page_table).cuda()
        ctx = torch.from_numpy(w.context_lens).cuda()

        # Outputs and workspace allocated once, outside the timed calls.
        out = torch.empty(workloads.query_shape(w), dtype=torch.float32, device="cuda")
        lse = torch.empty(w.batch, 1, w.hq, dtype=torch.float32, device="cuda")
        dargs, _ = atlas.make_attn_args(q, k, v, pt, ctx, w.scale)
        ws = torch.empty(max(1, atlas.atlas_decode_workspace_bytes(dargs)), dtype=torch.uint8, device="cuda")

        def call():
            if cold is not None:
                atlas.atlas_regenerate_pages(k, v, cold, seed=w.seed, layer=w.layer)
            return atlas.atlas_attend_decode(q, k, v, pt, ctx, w.scale, out=out, lse=lse, workspace=ws)[0]
        r = rep.setdefault("single_head_decode", {})
        med, mn = _call_stats_us(torch, np, call)
        r[f"{mode}_us"], r[f"{mode}_us_min"] = round(med, 2), round(mn, 2)
        if mode == "resident":
            r["c_abi_us"] = round(_c_abi_call_us(torch, np, "atlas_attend_decode", atlas.make_attn_args(
                q, k, v, pt, ctx, w.scale, out=out, lse=lse, workspace=ws)[0], calls=50), 2)
            prep = atlas.prepare_attend("decode", q, k, v, pt, ctx, w.scale, out=out, lse=lse, workspace=ws)
            r["prepared_us"] = round(_median_call_us(torch, np, prep, calls=50), 2)
            r["graph10_us"] = round(_graph10_us(torch, np, prep), 2)
            if oracle is not None:
                r["cpu_baseline"] = _oracle_single_head(w, q, out, np, oracle)
    kvb = int(w.context_lens.sum()) * w.hkv * w.head_dim * 4 * 2
    us = rep["single_head_decode"]["resident_us"]
    rep["single_head_decode"].update({"kv_bytes": kvb, "GBs": round(kvb / us / 1e3, 1),
                                      "frac_hbm": round(kvb / us / 1e3 / HBM_PEAK_GBS, 4),
                                      "note": "launch-latency bound (2 MiB of K/V); *_us are per Python "
                                              "call, host overhead included (c_abi_us: one C-ABI call with "
                                              "prepared arguments; prepared_us: a prepare_attend call from "
                                              "Python; graph10_us: per call in a HIP graph of ten); cold "
                                              "regenerates all 8 pages in the call"})
    # GQA short-query suffix attention (16 queries at positions 240..255).
    w = workloads.make("gqa_short_query")
    lay = workloads.page_layout(w)
    k, v = _arena(torch, workloads, np, w, lay)
    q = workloads.randn(workloads.query_shape(w), seed=w.seed * 100 + 1, device="cuda")
    pt = torch.from_numpy(lay.page_table).cuda()
    ctx = torch.from_numpy(w.context_lens).cuda()
    out = torch.empty(workloads.query_shape(w), dtype=torch.float32, device="cuda")
    lse = torch.empty(w.batch, w.q_len, w.hq, dtype=torch.float32, device="cuda")
    pargs, _ = atlas.make_attn_args(q, k, v, pt, ctx, w.scale)
    ws = torch.empty(max(1, atlas.atlas_prefill_workspace_bytes(pargs)), dtype=torch.uint8, device="cuda")
    call = lambda: atlas.atlas_attend_prefill(q, k, v, pt, ctx, w.scale, out=out, lse=lse, workspace=ws)[0]
    us, us_min = _call_stats_us(torch, np, call)
    c_us = _c_abi_call_us(torch, np, "atlas_attend_prefill", atlas.make_attn_args(
        q, k, v, pt, ctx, w.scale, out=out, lse=lse, workspace=ws)[0], calls=50)
    prep = atlas.prepare_attend("prefill", q, k, v, pt, ctx, w.scale, out=out, lse=lse, workspace=ws)
    p_us = _median_call_us(torch, np, prep, calls=50)
    g_us = _graph10_us(torch, np, prep)
    L = int(w.context_lens[0])
    pairs = w.hq * sum(L - w.q_len + i + 1 for i in range(w.q_len))
    rep["gqa_short_query"] = {"us": round(us, 2), "us_min": round(us_min, 2), "c_abi_us": round(c_us, 2),
                              "prepared_us": round(p_us, 2), "graph10_us": round(g_us, 2),
                              "kv_bytes": L * w.hkv * w.head_dim * 4 * 2,
                              "flop": 4 * w.head_dim * pairs,
                              "note": "latency bound (256 KiB of K/V); us per Python call, host overhead included; "
                                      "c_abi_us: one C-ABI call with prepared arguments; prepared_us: a "
                                      "prepare_attend call from Python; graph10_us: per call in a HIP graph "
                                      "of ten"}
    if oracle is not None:
        rep["gqa_short_query"]["cpu_baseline"] = _oracle_short_query(w, lay, q, k, v, out, np, oracle, pairs)
    del k, v
    # Mixed-length decode with window / sinks / softcap on even sequences.
    w = workloads.make("mixed_decode")
    lay = workloads.page_layout(w)
    k, v = _arena(torch, workloads, np, w, lay)
    q = workloads.randn(workloads.query_shape(w), seed=w.seed * 100 + 1, dtype=w.dtype, device="cuda")
    pt = torch.from_numpy(lay.page_table).cuda()
    ctx = torch.from_numpy(w.context_lens).cuda()
    opt = lambda a, t: torch.from_numpy(a.astype(t)).cuda()
    win, snk, cap = opt(w.window, np.int32), opt(w.sinks, np.int32), opt(w.softcap, np.float32)
    out = torch.empty(workloads.query_shape(w), dtype=torch.float32, device="cuda")
    us, us_min = _call_stats_us(torch, np, lambda: atlas.atlas_attend_decode(
        q, k, v, pt, ctx, w.scale, window=win, sink_tokens=snk, softcap=cap, out=out))
    Ls = w.context_lens.astype(np.int64)
    Ws = w.window.astype(np.int64)
    Ss = w.sinks.astype(np.int64)
    vis = np.where(Ws > 0, np.minimum(Ws, Ls) + np.minimum(Ss, np.maximum(Ls - Ws, 0)), Ls)
    kvb = int(vis.sum()) * w.hkv * w.head_dim * 2 * 2
    rep["mixed_decode"] = {"us": round(us, 1), "us_min": round(us_min, 1), "kv_bytes": kvb,
                           "GBs": round(kvb / us / 1e3, 1), "frac_hbm": round(kvb / us / 1e3 / HBM_PEAK_GBS, 4),
                           "note": "visible-key bytes (window + sinks on even sequences)"}
    if oracle is not None:
        rep["mixed_decode"]["cpu_baseline"] = _oracle_mixed_decode(torch, w, lay, q, k, v, out, vis, np, oracle)
    del k, v
    torch.cuda.empty_cache()
    return rep


def _oracle_single_head(w, q, out, np, oracle, min_seconds=1.0):
    """The oracle on the whole single-head decode (4096 keys, K/V from its own
    generator, generation untimed), in KV GB/s."""
    L = int(w.context_lens[0])
    k = np.stack([oracle.regen_rows(w.seed, w.layer, 0, oracle.TENSOR_K, h, 0, L, w.head_dim) for h in range(w.hkv)])
    v = np.stack([oracle.regen_rows(w.seed, w.layer, 0, oracle.TENSOR_V, h, 0, L, w.head_dim) for h in range(w.hkv)])
    qh = q[0].cpu().numpy()
    hm = oracle.default_head_map(w.hq, w.hkv)
    pos = np.array([L - 1], np.int32)
    ro, _ = oracle.attend(qh, k, v, pos, hm, w.scale)
    err = np.abs(out[0].cpu().numpy().astype(np.float64) - ro)
    if not np.all(err <= 2e-5 + 1e-4 * np.abs(ro)):
        raise SystemExit(f"bench: GPU single-head decode disagrees with the oracle (max err {err.max():.3e})")
    n, secs = _oracle_timed(lambda: oracle.attend(qh, k, v, pos, hm, w.scale), min_seconds)
    kvb = k.nbytes + v.nbytes
    return {"value": round(n * kvb / secs / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(),
            "cpu_model": _cpu_model(), "kind": "oracle",
            "sample": f"whole workload (1 row x {L} keys, {kvb / 2**20:.0f} MiB fp32 K/V) x {n} calls, "
                      f"{secs:.2f} s timed; K/V generation untimed; GPU output agreed (max abs err {err.max():.2e})"}


def _oracle_short_query(w, lay, q, k_dev, v_dev, out, np, oracle, pairs, min_seconds=1.0):
    """The oracle on the whole GQA short query (K/V read back from the arena
    through the page table), in GFLOP/s over the visible pairs."""
    L = int(w.context_lens[0])
    k = oracle.gather_pages(k_dev.cpu().numpy(), lay.page_table[0], L, w.page_size)
    v = oracle.gather_pages(v_dev.cpu().numpy(), lay.page_table[0], L, w.page_size)
    qh = q[0].cpu().numpy()
    hm = oracle.default_head_map(w.hq, w.hkv)
    pos = np.arange(L - w.q_len, L, dtype=np.int32)
    ro, _ = oracle.attend(qh, k, v, pos, hm, w.scale)
    err = np.abs(out[0].cpu().numpy().astype(np.float64) - ro)
    if not np.all(err <= 2e-5 + 1e-4 * np.abs(ro)):
        raise SystemExit(f"bench: GPU short-query output disagrees with the oracle (max err {err.max():.3e})")
    n, secs = _oracle_timed(lambda: oracle.attend(qh, k, v, pos, hm, w.scale), min_seconds)
    flop = 4.0 * w.head_dim * pairs
    return {"value": round(n * flop / secs / 1e9, 3), "unit": "GFLOP/s", "cores": oracle.num_threads(),
            "cpu_model": _cpu_model(), "kind": "oracle",
            "sample": f"whole workload ({w.q_len} queries x {w.hq} q-heads over {L} keys, {flop / 1e6:.2f} MFLOP) "
                      f"x {n} calls, {secs:.2f} s timed; GPU output agreed (max abs err {err.max():.2e})"}


def _oracle_mixed_decode(torch, w, lay, q, k_dev, v_dev, out, vis, np, oracle, seqs=(0, 1, 2, 3),
                         min_seconds=1.0):
    """The oracle on a sample of the mixed-length decode (sequences `seqs`:
    windowed and plain ones), K/V read back from the arena through the page
    table, in KV GB/s over those sequences' visible-key bytes (bf16, as the
    GPU figure counts them)."""
    P, D = w.page_size, w.head_dim
    hm = oracle.default_head_map(w.hq, w.hkv)
    o = out.cpu().numpy()
    qh = q.float().cpu().numpy()
    secs, kvb, max_err, lens = 0.0, 0, 0.0, []
    for b in seqs:
        L = int(w.context_lens[b])
        n_pages = (L + P - 1) // P
        ids = torch.from_numpy(lay.page_table[b, :n_pages].astype(np.int64)).cuda()
        k = k_dev.index_select(0, ids).float().permute(1, 0, 2, 3).reshape(w.hkv, n_pages * P, D)[:, :L]
        v = v_dev.index_select(0, ids).float().permute(1, 0, 2, 3).reshape(w.hkv, n_pages * P, D)[:, :L]
        k, v = np.ascontiguousarray(k.cpu().numpy()), np.ascontiguousarray(v.cpu().numpy())
        win, snk, cap = int(w.window[b]), int(w.sinks[b]), float(w.softcap[b])
        pos = np.array([L - 1], np.int32)
        ro, _ = oracle.attend(qh[b], k, v, pos, hm, w.scale, win, snk if win > 0 else 0, cap)
        err = np.abs(o[b].astype(np.float64) - ro)
        if not np.all(err <= 2e-3):
            raise SystemExit(f"bench: GPU mixed decode disagrees with the oracle (seq {b}, max err {err.max():.3e})")
        max_err = max(max_err, float(err.max()))
        n, t = _oracle_timed(lambda: oracle.attend(qh[b], k, v, pos, hm, w.scale, win, snk if win > 0 else 0, cap),
                             min_seconds / len(seqs))
        secs += t / n
        kvb += int(vis[b]) * w.hkv * D * 2 * 2
        lens.append(L)
        del k, v
    return {"value": round(kvb / secs / 1e9, 3), "unit": "GB/s", "cores": oracle.num_threads(),
            "cpu_model": _cpu_model(), "kind": "oracle",
            "sample": f"sequences {list(seqs)} of 64 (lengths {lens}; even ones windowed), "
                      f"{kvb / 1e6:.1f} MB of visible bf16 K/V per pass, each timed over >= "
                      f"{min_seconds / len(seqs):.2f} s; GPU outputs agreed (max abs err {max_err:.2e})"}


def cpu_baseline(d, out, np, oracle, min_seconds=3.0):
    """Time the oracle's attention (fp64 two-pass, OpenMP) on the decode
    workload: all 8 sequences x 32 q-heads x 65536 keys, repeated until at
    least `min_seconds` of timed work.  K/V come from the oracle's own
    generator and that generation is not timed (the GPU figure it is compared
    with excludes regeneration too).  The GPU outputs are checked against the
    oracle's on the way."""
    w = d["w"]
    q = d["q"].cpu().numpy()
    hm = oracle.default_head_map(w.hq, w.hkv)
    kv = []
    for b in range(w.batch):
        L = int(w.context_lens[b])
        kk = np.stack([oracle.regen_rows(w.seed, w.layer, b, oracle.TENSOR_K, h, 0, L, w.head_dim)
                       for h in range(w.hkv)])
        vv = np.stack([oracle.regen_rows(w.seed, w.layer, b, oracle.TENSOR_V, h, 0, L, w.head_dim)
                       for h in range(w.hkv)])
        kv.append((kk, vv))
    bytes_per_pass = sum(kk.nbytes + vv.nbytes for kk, vv in kv)
    secs, passes, max_err = 0.0, 0, 0.0
    while secs < min_seconds:
        for b, (kk, vv) in enumerate(kv):
            L = int(w.context_lens[b])
            t0 = time.perf_counter()
            ro, _ = oracle.attend(q[b], kk, vv, np.array([L - 1], np.int32), hm, w.scale)
            secs += time.perf_counter() - t0
            if passes == 0:
                err = np.abs(out[b].astype(np.float64) - ro)
                if not np.all(err <= 2e-5 + 1e-4 * np.abs(ro)):
                    raise SystemExit(f"bench: GPU decode output disagrees with the oracle "
                                     f"(seq {b}, max err {err.max():.3e})")
                max_err = max(max_err, float(err.max()))
        passes += 1
    return {"value": round(passes * bytes_per_pass / secs / 1e9, 3), "unit": "GB/s",
            "cores": oracle.num_threads(), "cpu_model": _cpu_model(), "kind": "oracle",
            "sample": f"whole decode workload (8 seqs x 32 q-heads x 65536 keys, "
                      f"{bytes_per_pass / 1e9:.2f} GB fp32 K/V) x {passes} passes, {secs:.2f} s timed; "
                      f"K/V generation untimed; GPU outputs agreed (max abs err {max_err:.2e})"}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _git_commit():
    try:
        r = subprocess.run(["git", "-C", os.path.dirname(os.path.abspath(__file__)), "rev-parse", "HEAD"],
                           capture_output=True, text=True, timeout=10)
        return r.stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        return None


def _rocm_version():
    for path in ("/opt/rocm/.info/version",):
        try:
            with open(path) as f:
                return f.read().strip()
        except OSError:
            pass
    return None


def gpu_sclk_mhz():
    """Current shader clock of GPU 0 as rocm-smi reports it (None if unavailable)."""
    try:
        r = subprocess.run(["rocm-smi", "-d", "0", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=20)
        data = json.loads(r.stdout)
    except (OSError, subprocess.SubprocessError, ValueError):
        return None
    for card in data.values():
        if isinstance(card, dict):
            for key, val in card.items():
                if "sclk" in key.lower():
                    m = re.search(r"(\d+)\s*Mhz", str(val), re.I)
                    if m:
                        return int(m.group(1))
    return None


def _library_build():
    """The library's build record (git commit and source hash at build time),
    and whether the sources here still hash the same."""
    here = os.path.dirname(os.path.abspath(__file__))
    try:
        with open(os.path.join(here, "exact_paged_causal_amd", "build_info.json")) as f:
            info = json.load(f)
    except (OSError, ValueError):
        return None
    import importlib.util
    spec = importlib.util.spec_from_file_location("_atlas_build", os.path.join(here, "exact_paged_causal_amd",
                                                                              "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    info["sources_unchanged_since_build"] = info.get("sources_sha256") == mod.sources_sha256()
    info.pop("hipcc_flags", None)
    return info


def provenance(torch):
    """Where the numbers come from (CPUAttn README, "Benchmark suite": reports
    carry their environment)."""
    prop = torch.cuda.get_device_properties(0)
    lib = _library_build()
    commit, source = _git_commit(), "git"
    if commit is None and lib:
        # a copy of the tree without its repository: the commit the library
        # was built at (library_build says whether the sources changed since)
        commit, source = lib.get("git_commit"), "library build record"
    return {"gpu": getattr(prop, "gcnArchName", None) or torch.cuda.get_device_name(0),
            "gpu_name": torch.cuda.get_device_name(0), "cu_count": prop.multi_processor_count,
            "gpu_sclk_mhz_after_timing": gpu_sclk_mhz(), "cpu_model": _cpu_model(),
            "host_threads": os.cpu_count(), "rocm": _rocm_version(), "hip_runtime": torch.version.hip,
            "torch": torch.__version__, "git_commit": commit, "git_commit_from": source, "library_build": lib}


def prefill_cpu_baseline(p, out, np, oracle, heads_per_kv=1, edge=512):
    """Time the oracle (fp64 two-pass, OpenMP) on a bounded sample of the
    8192-token causal prefill: every row of one q-head per K/V head (8 of the
    32) plus the first and last `edge` rows of every q-head, in GFLOP/s over
    that sample's visible pairs (4 D flop per pair, as for the GPU figure).
    The GPU output is checked against the oracle's on the same rows."""
    w = p["w"]
    S, D = w.q_len, w.head_dim
    P = w.page_size
    n_pages = S // P
    kl = p["kl"].float().cpu().numpy()[:n_pages]       # logical pages [n][Hkv][P][D]
    vl = p["vl"].float().cpu().numpy()[:n_pages]
    k = np.ascontiguousarray(kl.transpose(1, 0, 2, 3).reshape(w.hkv, S, D))
    v = np.ascontiguousarray(vl.transpose(1, 0, 2, 3).reshape(w.hkv, S, D))
    q = p["q"][0].float().cpu().numpy()                  # [S][Hq][D]
    o = out[0]
    hm = oracle.default_head_map(w.hq, w.hkv)
    heads = np.array([g * (w.hq // w.hkv) for g in range(w.hkv)])
    ends = np.array(sorted(set(range(edge)) | set(range(S - edge, S))))
    blocks = [(np.arange(S), heads), (ends, np.arange(w.hq))]
    flop, secs, max_err = 0.0, 0.0, 0.0
    for rows, hs in blocks:
        qq = np.ascontiguousarray(q[rows][:, hs])
        t0 = time.perf_counter()
        ro, _ = oracle.attend(qq, k, v, rows.astype(np.int32), hm[hs], w.scale)
        secs += time.perf_counter() - t0
        flop += 4.0 * D * len(hs) * float((rows + 1).sum())
        err = np.abs(o[rows][:, hs].astype(np.float64) - ro)
        if not np.all(err <= 2e-3):
            raise SystemExit(f"bench: GPU prefill output disagrees with the oracle (max err {err.max():.3e})")
        max_err = max(max_err, float(err.max()))
    return {"value": round(flop / secs / 1e9, 3), "unit": "GFLOP/s", "cores": oracle.num_threads(),
            "cpu_model": _cpu_model(), "kind": "oracle",
            "sample": f"every row of {len(heads)} q-heads (one per K/V head) + the first and last {edge} rows of "
                      f"all {w.hq} q-heads of the 8192-token prefill: {flop / 1e9:.1f} GFLOP over visible pairs, "
                      f"{secs:.2f} s timed; GPU outputs agreed (max abs err {max_err:.2e})"}


def main():
    args = parse()
    REPORT_WARMUP[:] = [max(0, args.report_warmup), max(0.0, args.report_warmup_s)]
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU; --gpus must be 1 (no multi-GPU path)"}))
        sys.exit(2)
    import numpy as np
    import torch

    import exact_paged_causal_amd as atlas
    import workloads

    torch.cuda.set_device(0)
    if args.workloads_only:
        print(json.dumps({"workloads": workload_report(torch, np, workloads, atlas), "n_gpus": 1}))
        return
    d = decode_setup(torch, workloads, atlas)
    w = d["w"]
    dec_out = torch.empty(workloads.query_shape(w), dtype=torch.float32, device="cuda")
    dec_lse = torch.empty(w.batch, 1, w.hq, dtype=torch.float32, device="cuda")
    args_tmp, _ = atlas.make_attn_args(d["q"], d["k"], d["v"], d["pt"], d["ctx"], w.scale,
                                       split_tokens=args.split_tokens)
    ws = torch.empty(atlas.atlas_decode_workspace_bytes(args_tmp), dtype=torch.uint8, device="cuda")

    p = None
    if not args.no_prefill:
        p = prefill_setup(torch, workloads, np)
        pw = p["w"]
        pre_out = torch.empty(workloads.query_shape(pw), dtype=torch.float32, device="cuda")
        pre_lse = torch.empty(pw.batch, pw.q_len, pw.hq, dtype=torch.float32, device="cuda")
        pargs, _ = atlas.make_attn_args(p["q"], p["k"], p["v"], p["pt"], p["ctx"], pw.scale)
        pws = torch.empty(atlas.atlas_prefill_workspace_bytes(pargs), dtype=torch.uint8, device="cuda")

    def regen():
        atlas.atlas_regenerate_pages(d["k"], d["v"], d["cold"], seed=w.seed, layer=w.layer)

    def decode():
        atlas.atlas_attend_decode(d["q"], d["k"], d["v"], d["pt"], d["ctx"], w.scale, out=dec_out,
                                  lse=dec_lse, workspace=ws, split_tokens=args.split_tokens)

    def prefill():
        atlas.atlas_attend_prefill(p["q"], p["k"], p["v"], p["pt"], p["ctx"], pw.scale, out=pre_out,
                                   lse=pre_lse, workspace=pws)

    # One step: regenerate the cold pages, run the prefill, then the decode
    # pass over hot + regenerated pages.  Prefill and decode are independent;
    # running the (compute-bound) prefill between the regenerator and the
    # decode pass lets the regenerated pages' write-back drain before the
    # decode pass streams them (with --no-prefill the decode pass follows
    # the regenerator directly).
    def step(t_regen=None, t_dec=None, t_pre=None):
        (t_regen or (lambda f: f()))(regen)
        if p is not None:
            (t_pre or (lambda f: f()))(prefill)
        (t_dec or (lambda f: f()))(decode)

    # The first (cold) step is timed on its own: first-call figures.
    f_regen, f_dec, f_pre = Timer(torch), Timer(torch), Timer(torch)
    step(f_regen, f_dec, f_pre)
    torch.cuda.synchronize()
    for _ in range(max(args.warmup - 1, 0)):
        step()
    torch.cuda.synchronize()
    print(f"bench: warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    t_regen, t_dec, t_pre = Timer(torch), Timer(torch), Timer(torch)
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    s0.record()
    for _ in range(args.steps):
        step(t_regen, t_dec, t_pre)
    s1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = s0.elapsed_time(s1) / args.steps
    dec_ms = float(np.median(t_dec.ms()))
    regen_ms = float(np.median(t_regen.ms()))
    print(f"bench: timed {args.steps} steps in {wall:.2f} s", file=sys.stderr, flush=True)
    if args.step_times:
        for name, t in (("regen", t_regen), ("prefill", t_pre), ("decode", t_dec)):
            if t.pairs:
                print(f"bench: {name} us per step: {[round(x * 1000) for x in t.ms()]}", file=sys.stderr, flush=True)

    kv_bytes = int(w.context_lens.astype(np.int64).sum()) * w.hkv * w.head_dim * 4 * 2
    dec_gbs = kv_bytes / (dec_ms * 1e-3) / 1e9
    n_cold = int(d["cold"].shape[0])
    regen_bytes = n_cold * w.hkv * w.page_size * w.head_dim * 4 * 2
    result = {
        "metric": METRIC,
        "value": round(dec_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "long_context_decode: B=8 x 65536 tokens, Hq=32, Hkv=8, D=64, page 512, fp32, "
                        "shuffled pool, 25% resident + 75% regenerated per step"
                        + ("" if p is None else "; causal_prefill: S=8192, Hq=32, Hkv=8, D=128, page 128, bf16"),
            "step_order": "regenerate, decode" if p is None else "regenerate, prefill, decode",
            "decode_attention_ms": round(dec_ms, 4),
            "decode_kv_bytes": kv_bytes,
            "regen_ms": round(regen_ms, 4),
            "regen_pages": n_cold,
            "regen_write_GBs": round(regen_bytes / (regen_ms * 1e-3) / 1e9, 1),
            "decode_end_to_end_ms": round(dec_ms + regen_ms, 4),
            "timing": "medians over the timed steps; min and the cold first step beside them",
            "decode_attention_ms_min": round(float(np.min(t_dec.ms())), 4),
            "regen_ms_min": round(float(np.min(t_regen.ms())), 4),
            "first_step_ms": {"decode_attention": round(f_dec.ms()[0], 4), "regen": round(f_regen.ms()[0], 4),
                              **({} if p is None else {"prefill": round(f_pre.ms()[0], 4)})},
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "decode attention pass (split-KV fold + LSE merge)",
            "achieved": round(dec_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("decode_split_long_context"),
            "traffic_unit": "HBM bytes per call (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
        },
    }
    if p is not None:
        pre_ms = float(np.median(t_pre.ms()))
        S, hq, dd = pw.q_len, pw.hq, pw.head_dim
        flops = 4.0 * dd * hq * S * (S + 1) / 2.0
        tf = flops / (pre_ms * 1e-3) / 1e12
        result["prefill"] = {
            "value": round(tf, 1), "unit": "TFLOP/s", "ms": round(pre_ms, 4),
            "ms_min": round(float(np.min(t_pre.ms())), 4), "flop": flops,
            "dtype": "bf16",
            "roofline": {"bound": "mfma", "kernel": "tiled causal prefill", "achieved": round(tf, 1),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("prefill_tiled_causal_8192"),
                         "traffic_unit": "HBM bytes per call (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"},
        }
    if not args.no_workloads:
        result["next"] = {"fused_regen_decode": fused_report(torch, np, d, atlas, dec_ms, regen_ms),
                          "append_kv": append_report(torch, np, workloads, atlas),
                          "hot_cache": cache_report(torch, np, workloads, atlas)}
        if p is not None:
            result["next"]["prefill_variants"] = prefill_variants_report(torch, np, p, atlas)
            result["next"]["prefill_f32"] = prefill_f32_report(torch, np, workloads, atlas)
            result["next"]["mods"] = mods_report(torch, np, p, atlas)
            result["next"]["chunked_prefill"] = chunked_prefill_report(torch, np, workloads, atlas)
            result["next"]["few_item"] = few_item_report(torch, np, workloads, atlas)
        print("bench: fused regeneration timed", file=sys.stderr, flush=True)
    if not args.no_workloads:
        # Every synthetic workload's throughput (the long-context decode and
        # the prefill are the step's own figures above).
        wl_oracle = None
        if not args.no_cpu_baseline:
            import oracle as wl_oracle
        wl = workload_report(torch, np, workloads, atlas, oracle=wl_oracle)
        wl["long_context_decode"] = {"us": round(dec_ms * 1000.0, 1), "kv_bytes": kv_bytes,
                                     "GBs": round(dec_gbs, 1), "frac_hbm": round(dec_gbs / HBM_PEAK_GBS, 4),
                                     "regen_us": round(regen_ms * 1000.0, 1)}
        if p is not None:
            wl["causal_prefill"] = {"us": round(pre_ms * 1000.0, 1), "flop": flops, "TFLOPs": round(tf, 1),
                                    "frac_mfma": round(tf / BF16_PEAK_TFLOPS, 4)}
        result["workloads"] = {k: wl[k] for k in ("single_head_decode", "gqa_short_query", "long_context_decode",
                                                  "causal_prefill", "mixed_decode") if k in wl}
        print("bench: workloads timed", file=sys.stderr, flush=True)
    # A plain 256 MiB device copy (the runtime's copy kernel) as context for
    # the HBM figures: bytes read + written per second.  The counter runs use
    # the same copy to calibrate FETCH_SIZE / WRITE_SIZE.
    src = torch.empty(1 << 28, dtype=torch.uint8, device="cuda")   # 256 MiB
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    tc = Timer(torch)
    for _ in range(10):
        tc(lambda: dst.copy_(src))
    torch.cuda.synchronize()
    cms = float(np.mean(tc.ms()))
    result["hbm_context"] = {"kernel": "256 MiB device-to-device copy", "bytes_read": src.numel(),
                             "bytes_written": dst.numel(), "ms": round(cms, 4),
                             "GBs_read_plus_written": round(2 * src.numel() / (cms * 1e-3) / 1e9, 1),
                             "frac_hbm": round(2 * src.numel() / (cms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del src, dst
    result["provenance"] = provenance(torch)
    if not args.no_cpu_baseline:
        import oracle
        result["cpu_baseline"] = cpu_baseline(d, dec_out.cpu().numpy(), np, oracle)
        print("bench: decode oracle baseline timed", file=sys.stderr, flush=True)
        if p is not None:
            result["prefill"]["cpu_baseline"] = prefill_cpu_baseline(p, pre_out.cpu().numpy(), np, oracle)
            print("bench: prefill oracle baseline timed", file=sys.stderr, flush=True)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

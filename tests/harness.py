"""Shared helpers for the GPU parity tests: device inputs from the seeded
workloads, the oracle's answer for the same inputs, and the tolerance check.

Tolerances (stated for this method): fp32 inputs |gpu - ref| <= 2e-5 +
1e-4 |ref| element-wise; bf16 inputs |gpu - ref| <= 2e-3 with fp32
accumulation.  Integer and index results are compared bit-exactly.

Regenerated bf16 K/V: the GPU's generator may differ from the exact value z
by up to GEN_BOUND (1 + |z|) before rounding to bf16, so an element whose z
lies that close to a bf16 rounding boundary may round to either neighbour.
For such workloads the bar adds, per output element, the first-order effect
of those elements, computed from the oracle's own values alone (see
regen_bf16_slack).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

import oracle
import workloads

F32_ATOL, F32_RTOL = 2e-5, 1e-4
BF16_ATOL = 2e-3
GEN_BOUND = 1e-6   # the GPU generator's error before rounding: |g - z| <= GEN_BOUND (1 + |z|)


def tdtype(w):
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def seq_keys_tensor(w, device="cuda"):
    """The workload's generator keys as a device tensor (None: batch rows)."""
    return None if w.seq_keys is None else torch.from_numpy(np.asarray(w.seq_keys, np.int32)).to(device)


def assert_close(got, want, dtype: str, what: str = "", extra=None):
    """Element-wise bar for the dtype; `extra` (broadcastable) is added to it."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    err = np.abs(got - want)
    bound = (F32_ATOL + F32_RTOL * np.abs(want)) if dtype == "f32" else np.full(want.shape, BF16_ATOL)
    if extra is not None:
        bound = bound + extra
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5].tolist()
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} out of tolerance, "
                             f"max err {np.nanmax(err):.3e}, first at {idx}: "
                             f"got {got[tuple(idx[0])]!r} want {want[tuple(idx[0])]!r}")


@dataclass
class DeviceInputs:
    w: workloads.Workload
    layout: workloads.PageLayout
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    page_table: torch.Tensor
    context_lens: torch.Tensor
    window: torch.Tensor | None
    sinks: torch.Tensor | None
    softcap: torch.Tensor | None
    cold_jobs: torch.Tensor | None
    hot_jobs: torch.Tensor | None


def logical_kv(w, device, seed_offset=0):
    """Seeded K/V in logical page order (see workloads.logical_kv)."""
    return workloads.logical_kv(w, device, seed_offset)


def build(w, device="cuda", hot_fraction=None, layout_seed=0, extra_phys=0, poison=False,
          regen_hot=True) -> DeviceInputs:
    """Device-resident inputs.  Regenerated workloads: resident pages are
    regenerated once here, cold pages are left for each call.  Others: seeded
    logical K/V scattered into a shuffled arena.  poison=True fills every
    arena row that no context covers (page tails, spare pages) with NaN."""
    import exact_paged_causal_amd as atlas
    lay = workloads.page_layout(w, hot_fraction, layout_seed, extra_phys)
    dt = tdtype(w)
    q = workloads.randn(workloads.query_shape(w), seed=w.seed * 100 + 1, dtype=w.qdt, device=device)
    shape = workloads.arena_shape(w, lay.num_phys)
    fill = float("nan") if poison else 0.0
    pt = torch.from_numpy(lay.page_table).to(device)
    ctx = torch.from_numpy(w.context_lens.astype(np.int32)).to(device)
    if w.regenerated:
        k = torch.full(shape, fill, dtype=dt, device=device)
        v = torch.full(shape, fill, dtype=dt, device=device)
        hot = torch.from_numpy(workloads.key_jobs(w, lay.hot_jobs)).to(device) if len(lay.hot_jobs) else None
        cold = torch.from_numpy(workloads.key_jobs(w, lay.cold_jobs)).to(device) if len(lay.cold_jobs) else None
        if regen_hot and hot is not None:
            atlas.atlas_regenerate_pages(k, v, hot, seed=w.seed, layer=w.layer)
    else:
        kl, vl, n_pages = logical_kv(w, device)
        k = torch.full(shape, fill, dtype=dt, device=device)
        v = torch.full(shape, fill, dtype=dt, device=device)
        ids = torch.from_numpy(np.concatenate([lay.page_table[b, :n_pages[b]]
                                               for b in range(w.batch)]).astype(np.int64)).to(device)
        k.index_copy_(0, ids, kl)
        v.index_copy_(0, ids, vl)
        del kl, vl
        if poison:
            # NaN in the rows past each context inside its last page
            for b in range(w.batch):
                L = int(w.context_lens[b])
                tail = L % w.page_size
                if tail:
                    pid = int(lay.page_table[b, (L - 1) // w.page_size])
                    k[pid, :, tail:, :] = float("nan")
                    v[pid, :, tail:, :] = float("nan")
        hot = cold = None
    opt = lambda a, t: None if a is None else torch.from_numpy(a.astype(t)).to(device)
    return DeviceInputs(w, lay, q, k, v, pt, ctx, opt(w.window, np.int32), opt(w.sinks, np.int32),
                        opt(w.softcap, np.float32), cold, hot)


def run(inp: DeviceInputs, entry: str | None = None, split_tokens: int = 0, workspace=None,
        head_map=None):
    """One call of the path: regenerate cold pages (if any), then attend."""
    import exact_paged_causal_amd as atlas
    w = inp.w
    if inp.cold_jobs is not None:
        atlas.atlas_regenerate_pages(inp.k, inp.v, inp.cold_jobs, seed=w.seed, layer=w.layer)
    if entry is None:
        entry = "decode" if w.q_len == 1 else "prefill"
    fn = atlas.atlas_attend_decode if entry == "decode" else atlas.atlas_attend_prefill
    return fn(inp.q, inp.k, inp.v, inp.page_table, inp.context_lens, w.scale,
              head_map=head_map, window=inp.window, sink_tokens=inp.sinks, softcap=inp.softcap,
              split_tokens=split_tokens, workspace=workspace)


def to_f32_numpy(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


class OracleSource:
    """Per-sequence unpaged K/V for the oracle: regenerated by the oracle's own
    generator, or gathered from a host copy of the arena through the page
    table."""

    def __init__(self, inp: DeviceInputs):
        self.inp = inp
        w = inp.w
        self.k_host = self.v_host = None
        if not w.regenerated:
            self.k_host = to_f32_numpy(inp.k)
            self.v_host = to_f32_numpy(inp.v)

    def kv(self, b: int):
        w = self.inp.w
        L = int(w.context_lens[b])
        if w.regenerated:
            kind = "f32" if w.dtype == "f32" else "bf16"
            ks, vs = [], []
            key = w.seq_key(b)
            for h in range(w.hkv):
                kr = oracle.regen_rows(w.seed, w.layer, key, oracle.TENSOR_K, h, 0, L, w.head_dim, kind)
                vr = oracle.regen_rows(w.seed, w.layer, key, oracle.TENSOR_V, h, 0, L, w.head_dim, kind)
                if kind == "bf16":
                    kr, vr = oracle.bf16_bits_to_f32(kr), oracle.bf16_bits_to_f32(vr)
                ks.append(kr)
                vs.append(vr)
            return np.stack(ks), np.stack(vs)
        pt = self.inp.layout.page_table[b]
        return (oracle.gather_pages(self.k_host, pt, L, w.page_size),
                oracle.gather_pages(self.v_host, pt, L, w.page_size))

    def kv_slack(self, b: int):
        """Regenerated bf16 K/V of sequence b: for each element, how far from
        the oracle's bf16 value the GPU's may land ([Hkv][L][D] each, zero
        where the rounding cannot change); None for other workloads."""
        w = self.inp.w
        if not (w.regenerated and w.dtype == "bf16"):
            return None
        L = int(w.context_lens[b])
        key = w.seq_key(b)
        out = []
        for tensor in (oracle.TENSOR_K, oracle.TENSOR_V):
            rows = []
            for h in range(w.hkv):
                z = oracle.regen_rows(w.seed, w.layer, key, tensor, h, 0, L, w.head_dim, "f64")
                rows.append(bf16_rounding_slack(z))
            out.append(np.stack(rows))
        return out[0], out[1]


def bf16_rne(x) -> np.ndarray:
    """fp32 values rounded to bf16 (nearest, ties to even), widened to fp64."""
    bits = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = (((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16) << 16).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)


def bf16_rounding_slack(z: np.ndarray) -> np.ndarray:
    """For exact values z: the largest |bf16(g) - bf16(fp32(z))| over the fp32
    values g within GEN_BOUND (1 + |z|) of z (rounding is monotone, so the
    two ends of that interval bound it); zero for most elements."""
    z = np.asarray(z, np.float64)
    e = GEN_BOUND * (1.0 + np.abs(z))
    b0 = bf16_rne(z.astype(np.float32))
    lo = bf16_rne((z - e).astype(np.float32))
    hi = bf16_rne((z + e).astype(np.float32))
    return np.maximum(np.abs(hi - b0), np.abs(lo - b0))


def regen_bf16_slack(inp, b, rows, head_map, src, heads, ref_o):
    """Extra bar for regenerated bf16 K/V (zero otherwise): with the oracle's
    softmax weights p over the visible keys, the first-order change of the
    output when elements round to their other neighbour is at most
    sum_j p_j dv_jd (values) plus sum_j p_j ds_j |v_jd - o_d| (keys, where
    ds_j = scale sum_d |q_d| dk_jd bounds the score's change; the softcap's
    slope is at most 1), and of lse at most sum_j p_j ds_j.  The key term is
    doubled to cover the second-order rest."""
    sl = src.kv_slack(b)
    if sl is None:
        return None, None
    dk, dv = sl
    w = inp.w
    k, v = src.kv(b)
    q = to_f32_numpy(inp.q[b]).astype(np.float64)
    L = int(w.context_lens[b])
    pos = np.arange(L - w.q_len, L)
    if rows is not None:
        q, pos = q[rows], pos[rows]
    hm = oracle.default_head_map(w.hq, w.hkv) if head_map is None else np.asarray(head_map, np.int32)
    if heads is not None:
        q, hm = q[:, heads], hm[heads]
    win = int(w.window[b]) if w.window is not None else 0
    snk = int(w.sinks[b]) if (w.sinks is not None and win > 0) else 0
    cap = float(w.softcap[b]) if w.softcap is not None else 0.0
    j = np.arange(L)
    vis = (j[None, :] <= pos[:, None]) & ((win <= 0) | (j[None, :] > pos[:, None] - win) | (j[None, :] < snk))
    tol_o = np.zeros(ref_o.shape)
    tol_l = np.zeros(ref_o.shape[:2])
    for hh in range(q.shape[1]):
        g = int(hm[hh])
        s = w.scale * (q[:, hh] @ k[g].astype(np.float64).T)             # [rows][L]
        if cap > 0.0:
            s = cap * np.tanh(s / cap)
        s = np.where(vis, s, -np.inf)
        mx = s.max(axis=1, keepdims=True)
        p = np.exp(s - np.where(np.isfinite(mx), mx, 0.0))
        p /= np.maximum(p.sum(axis=1, keepdims=True), np.finfo(np.float64).tiny)
        ds = w.scale * (np.abs(q[:, hh]) @ dk[g].T)                       # [rows][L]
        pds = p * ds
        vk = v[g].astype(np.float64)
        tol_o[:, hh] = p @ dv[g] + 2.0 * (pds @ np.abs(vk)
                                          + pds.sum(axis=1, keepdims=True) * np.abs(ref_o[:, hh]))
        tol_l[:, hh] = 2.0 * pds.sum(axis=1)
    return tol_o, tol_l


def oracle_answer(inp: DeviceInputs, b: int, rows=None, head_map=None, src: OracleSource | None = None,
                  heads=None):
    """Oracle output for sequence b (all query rows, or the listed ones; all
    q-heads, or the listed ones)."""
    w = inp.w
    src = src or OracleSource(inp)
    k, v = src.kv(b)
    q = to_f32_numpy(inp.q[b])                       # [q_len][Hq][D]
    L = int(w.context_lens[b])
    pos = np.arange(L - w.q_len, L, dtype=np.int32)
    if rows is not None:
        q, pos = q[rows], pos[rows]
    hm = oracle.default_head_map(w.hq, w.hkv) if head_map is None else np.asarray(head_map, np.int32)
    if heads is not None:
        q, hm = np.ascontiguousarray(q[:, heads]), hm[heads]
    win = int(w.window[b]) if w.window is not None else 0
    snk = int(w.sinks[b]) if (w.sinks is not None and win > 0) else 0
    cap = float(w.softcap[b]) if w.softcap is not None else 0.0
    return oracle.attend(q, k, v, pos, hm, w.scale, win, snk, cap)


def check_against_oracle(inp, out, lse, seqs=None, rows=None, head_map=None, what="", heads=None):
    w = inp.w
    src = OracleSource(inp)
    out_h = to_f32_numpy(out)
    lse_h = to_f32_numpy(lse) if lse is not None else None
    for b in (range(w.batch) if seqs is None else seqs):
        ref_o, ref_l = oracle_answer(inp, b, rows, head_map, src, heads)
        tol_o, tol_l = regen_bf16_slack(inp, b, rows, head_map, src, heads, ref_o)
        got_o = out_h[b] if rows is None else out_h[b][rows]
        got_o = got_o if heads is None else got_o[:, heads]
        assert_close(got_o, ref_o, w.dtype, f"{what} out[b={b}]", tol_o)
        if lse_h is not None:
            got_l = lse_h[b] if rows is None else lse_h[b][rows]
            got_l = got_l if heads is None else got_l[:, heads]
            assert_close(got_l, ref_l, w.dtype, f"{what} lse[b={b}]", tol_l)


def full_size_blocks(w, seed: int, edge: int = 512):
    """(rows, heads) blocks the oracle checks on a full-size prefill it cannot
    afford whole: every row of one seeded q-head per K/V head, and the first
    and last `edge` rows of every q-head."""
    rng = np.random.default_rng(seed)
    hm = oracle.default_head_map(w.hq, w.hkv)
    heads = np.array(sorted(int(rng.choice(np.flatnonzero(hm == g))) for g in range(w.hkv)))
    n = w.q_len
    ends = np.array(sorted(set(range(min(edge, n))) | set(range(max(0, n - edge), n))))
    return [(np.arange(n), heads), (ends, np.arange(w.hq))]

"""GPU tests of K/V append, the page pool and shared prefix pages, through
the C ABI: appended rows land bit for bit where the page table says and
nowhere else; a decode stream that grows one token per step matches the fp64
oracle at every step; sequences that share a prefix's pages match the oracle
on their own logical histories.

Each test prints the case it runs before touching the GPU."""
import math

import numpy as np
import pytest
import torch

import harness as H
import oracle
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


TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128), ("f32", 128)])
def test_append_writes_exactly_the_target_rows(dtype, d):
    import exact_paged_causal_amd as atlas
    B, n_new, hkv, P, phys, maxp = 3, 21, 2, 16, 20, 6
    say(f"[append] {dtype} D={d}")
    k = workloads.randn((phys, hkv, P, d), seed=41, dtype=dtype, device="cuda")
    v = workloads.randn((phys, hkv, P, d), seed=42, dtype=dtype, device="cuda")
    kn = workloads.randn((B, n_new, hkv, d), seed=43, dtype=dtype, device="cuda")
    vn = workloads.randn((B, n_new, hkv, d), seed=44, dtype=dtype, device="cuda")
    rng = np.random.default_rng(7)
    pt = rng.permutation(phys)[:B * maxp].reshape(B, maxp).astype(np.int32)   # distinct pages
    start = np.array([0, 15, 70], np.int32)            # page-aligned, crossing pages, ends at 90 < 96
    exp_k, exp_v = k.clone(), v.clone()
    for b in range(B):
        for t in range(n_new):
            p = int(start[b]) + t
            exp_k[pt[b, p // P], :, p % P, :] = kn[b, t]
            exp_v[pt[b, p // P], :, p % P, :] = vn[b, t]
    atlas.atlas_append_kv(k, v, kn, vn, torch.from_numpy(pt).cuda(), torch.from_numpy(start).cuda())
    torch.cuda.synchronize()
    assert torch.equal(k, exp_k) and torch.equal(v, exp_v)


def test_append_skips_rows_outside_the_pool_and_validation_rejects_them(monkeypatch):
    import exact_paged_causal_amd as atlas
    P, hkv, d = 16, 1, 64
    say("[append] invalid page ids")
    k = torch.zeros((4, hkv, P, d), device="cuda")
    v = torch.zeros_like(k)
    kn = torch.ones((1, 20, hkv, d), device="cuda")
    vn = torch.ones_like(kn)
    pt = torch.tensor([[2, -5, 1]], dtype=torch.int32, device="cuda")   # positions 16..31 have no page
    sp = torch.tensor([0], dtype=torch.int32, device="cuda")
    monkeypatch.setenv("ATLAS_VALIDATE", "0")                        # also when the suite runs validated
    atlas.atlas_append_kv(k, v, kn, vn, pt, sp)
    torch.cuda.synchronize()
    assert torch.all(k[2] == 1) and int((k != 0).sum()) == P * d     # page 2 only
    monkeypatch.setenv("ATLAS_VALIDATE", "1")
    say("[append] validation mode")
    k.zero_()
    with pytest.raises(atlas.AtlasError) as ei:
        atlas.atlas_append_kv(k, v, kn, vn, pt, sp)
    assert ei.value.status == atlas.ATLAS_ERR_POOL
    with pytest.raises(atlas.AtlasError) as ei:                        # positions past the table
        atlas.atlas_append_kv(k, v, kn, vn, pt, torch.tensor([40], dtype=torch.int32, device="cuda"))
    assert ei.value.status == atlas.ATLAS_ERR_RANGE
    torch.cuda.synchronize()
    assert int((k != 0).sum()) == 0                                   # nothing was written


def _check_seq(out, lse, q, kk, vv, L, hm, scale, dtype, what):
    ro, rl = oracle.attend(q, kk[:, :L], vv[:, :L], np.array([L - 1], np.int32), hm, scale)
    H.assert_close(out, ro, dtype, what)
    H.assert_close(lse, rl, dtype, what + " lse")


def test_growing_decode_stream_matches_oracle():
    """Two sequences decode 6 steps; each step appends the new token's K/V
    (allocating a page from the pool when it crosses into a new one) and
    attends over the grown history."""
    import exact_paged_causal_amd as atlas
    B, hq, hkv, d, P, maxp = 2, 8, 2, 64, 16, 16
    scale = 1.0 / math.sqrt(d)
    hm = np.arange(hq) // (hq // hkv)
    pool = atlas.PagePool(2 * maxp)
    k = torch.full((2 * maxp, hkv, P, d), float("nan"), device="cuda")   # unwritten rows are never read
    v = torch.full_like(k, float("nan"))
    lens = [37, 95]
    total = [L + 6 for L in lens]
    # logical histories on the host: [hkv][L][D] per sequence
    kk = [workloads.randn((hkv, T, d), seed=50 + b).numpy() for b, T in enumerate(total)]
    vv = [workloads.randn((hkv, T, d), seed=60 + b).numpy() for b, T in enumerate(total)]
    pt = np.zeros((B, maxp), np.int32)
    for b, L in enumerate(lens):
        pt[b, :(L + P - 1) // P] = pool.alloc((L + P - 1) // P)
    ptd = torch.from_numpy(pt).cuda()
    say("[stream] initial histories")
    for b, L in enumerate(lens):
        kn = torch.from_numpy(np.ascontiguousarray(kk[b][:, :L].transpose(1, 0, 2)))[None].cuda()
        vn = torch.from_numpy(np.ascontiguousarray(vv[b][:, :L].transpose(1, 0, 2)))[None].cuda()
        atlas.atlas_append_kv(k, v, kn, vn, ptd[b:b + 1], torch.tensor([0], dtype=torch.int32, device="cuda"))
    for step in range(6):
        say(f"[stream] step {step}")
        for b in range(B):
            p = lens[b]
            if p % P == 0:                                  # the new token opens a page
                pt[b, p // P] = pool.alloc(1)[0]
        ptd = torch.from_numpy(pt).cuda()
        kn = torch.from_numpy(np.stack([kk[b][:, lens[b]] for b in range(B)]))[:, None].cuda()
        vn = torch.from_numpy(np.stack([vv[b][:, lens[b]] for b in range(B)]))[:, None].cuda()
        atlas.atlas_append_kv(k, v, kn, vn, ptd, torch.tensor(lens, dtype=torch.int32, device="cuda"))
        lens = [L + 1 for L in lens]
        q = workloads.randn((B, 1, hq, d), seed=70 + step, device="cuda")
        out, lse = atlas.atlas_attend_decode(q, k, v, ptd, torch.tensor(lens, dtype=torch.int32, device="cuda"),
                                             scale)
        torch.cuda.synchronize()
        for b in range(B):
            _check_seq(out[b].cpu().numpy(), lse[b].cpu().numpy(), q[b].cpu().numpy(), kk[b], vv[b], lens[b],
                       hm, scale, "f32", f"stream step {step} seq {b}")
    used = sum((L + P - 1) // P for L in lens)
    assert pool.free_pages() == 2 * maxp - used


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_shared_prefix_pages(dtype):
    """Three sequences share a 48-token prefix (three full pages, one copy in
    the arenas, reference count 3); each appends its own suffix into its own
    pages.  Decode and prefill over each history match the oracle, before and
    after one of the sequences releases its pages."""
    import exact_paged_causal_amd as atlas
    hq, hkv, d, P, maxp, n_pre = 8, 2, 128, 16, 8, 48
    scale = 1.0 / math.sqrt(d)
    hm = np.arange(hq) // (hq // hkv)
    pool = atlas.PagePool(24)
    k = torch.full((24, hkv, P, d), float("nan"), dtype=TORCH[dtype], device="cuda")
    v = torch.full_like(k, float("nan"))
    pre_k = workloads.randn((1, n_pre, hkv, d), seed=80, dtype=dtype, device="cuda")
    pre_v = workloads.randn((1, n_pre, hkv, d), seed=81, dtype=dtype, device="cuda")
    shared = pool.alloc(n_pre // P)
    pool.retain(shared)
    pool.retain(shared)
    assert [pool.refcount(i) for i in shared] == [3, 3, 3]
    suffix = [5, 30, 17]
    B = len(suffix)
    pt = np.zeros((B, maxp), np.int32)
    for b, s in enumerate(suffix):
        pt[b, :n_pre // P] = shared
        pt[b, n_pre // P:n_pre // P + (s + P - 1) // P] = pool.alloc((s + P - 1) // P)
    ptd = torch.from_numpy(pt).cuda()
    say(f"[prefix] {dtype}: prefix written once")
    atlas.atlas_append_kv(k, v, pre_k, pre_v, ptd[0:1], torch.tensor([0], dtype=torch.int32, device="cuda"))
    suf_k, suf_v = [], []
    for b, s in enumerate(suffix):
        sk = workloads.randn((1, s, hkv, d), seed=90 + b, dtype=dtype, device="cuda")
        sv = workloads.randn((1, s, hkv, d), seed=95 + b, dtype=dtype, device="cuda")
        atlas.atlas_append_kv(k, v, sk, sv, ptd[b:b + 1], torch.tensor([n_pre], dtype=torch.int32, device="cuda"))
        suf_k.append(sk)
        suf_v.append(sv)
    lens = [n_pre + s for s in suffix]
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")

    def logical(b):
        kk = torch.cat([pre_k[0], suf_k[b][0]]).float().permute(1, 0, 2).cpu().numpy()
        vv = torch.cat([pre_v[0], suf_v[b][0]]).float().permute(1, 0, 2).cpu().numpy()
        return kk, vv

    def check(seqs, what):
        q = workloads.randn((B, 1, hq, d), seed=99, dtype=dtype, device="cuda")
        out, lse = atlas.atlas_attend_decode(q, k, v, ptd, ctx, scale)
        qp = workloads.randn((B, 4, hq, d), seed=98, dtype=dtype, device="cuda")
        outp, lsep = atlas.atlas_attend_prefill(qp, k, v, ptd, ctx, scale)
        torch.cuda.synchronize()
        for b in seqs:
            kk, vv = logical(b)
            L = lens[b]
            _check_seq(out[b].cpu().numpy(), lse[b].cpu().numpy(), q[b].float().cpu().numpy(), kk, vv, L, hm,
                       scale, dtype, f"{what} decode seq {b}")
            ro, rl = oracle.attend(qp[b].float().cpu().numpy(), kk, vv, np.arange(L - 4, L, dtype=np.int32), hm,
                                   scale)
            H.assert_close(outp[b].cpu().numpy(), ro, dtype, f"{what} prefill seq {b}")

    check(range(B), "shared")
    say(f"[prefix] {dtype}: sequence 1 releases its pages")
    own1 = [int(x) for x in pt[1, n_pre // P:n_pre // P + (suffix[1] + P - 1) // P]]
    pool.release(shared + own1)
    assert [pool.refcount(i) for i in shared] == [2, 2, 2] and all(pool.refcount(i) == 0 for i in own1)
    check([0, 2], "after release")

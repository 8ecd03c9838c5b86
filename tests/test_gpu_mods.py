"""GPU parity of atlas_attend_mods (non-causal rows, ALiBi slopes, mask bits)
against the fp64 oracle, through the C ABI, on the split-KV kernels
(q_len < 64 and decode) and the tiled prefill kernels (q_len >= 64, bf16 and
fp32).  Rows with nothing visible must come back NaN with lse = -inf.  Each
test prints its case before running."""
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


def alibi_slopes(hq):
    """The geometric ALiBi slopes 2^(-8 (h + 1) / Hq)."""
    return (2.0 ** (-8.0 * (np.arange(hq) + 1) / hq)).astype(np.float32)


def pack_mask(mask, words):
    """[B][q_len][n] booleans -> [B][q_len][words] int32, bit j & 31 of word
    j >> 5 = key j."""
    B, nq, n = mask.shape
    bits = np.zeros((B, nq, words * 32), bool)
    bits[..., :n] = mask
    packed = np.packbits(bits, axis=-1, bitorder="little")
    return torch.from_numpy(np.ascontiguousarray(packed).view("<u4").astype(np.uint32).view(np.int32)).cuda()


def make_mask(w, density, seed, empty_rows=0):
    """Random keep-mask over every row's keys, each row's own position kept;
    the first `empty_rows` rows of sequence 0 hide everything."""
    L = int(w.page_size * ((int(w.context_lens.max()) + w.page_size - 1) // w.page_size))
    rng = np.random.default_rng(seed)
    m = rng.random((w.batch, w.q_len, L)) < density
    for b in range(w.batch):
        ctx = int(w.context_lens[b])
        m[b, np.arange(w.q_len), ctx - w.q_len + np.arange(w.q_len)] = True
    if empty_rows:
        m[0, :empty_rows] = False
    return m


def run_mods(inp, causal, slopes, mask):
    import exact_paged_causal_amd as atlas
    w = inp.w
    max_ctx = int(inp.layout.page_table.shape[1]) * w.page_size
    words = (max_ctx + 31) // 32
    return atlas.atlas_attend_mods(
        inp.q, inp.k, inp.v, inp.page_table, inp.context_lens, w.scale, causal=causal,
        alibi_slopes=None if slopes is None else torch.from_numpy(slopes).cuda(),
        mask_bits=None if mask is None else pack_mask(mask, words),
        window=inp.window, sink_tokens=inp.sinks, softcap=inp.softcap)


def check_mods(inp, out, lse, causal, slopes, mask, what, rows=None, heads=None):
    w = inp.w
    src = H.OracleSource(inp)
    out_h, lse_h = H.to_f32_numpy(out), H.to_f32_numpy(lse)
    hsel = np.arange(w.hq) if heads is None else np.asarray(heads)
    hm = oracle.default_head_map(w.hq, w.hkv)[hsel]
    if slopes is not None:
        slopes = slopes[hsel]
    for b in range(w.batch):
        k, v = src.kv(b)
        L = int(w.context_lens[b])
        sel = np.arange(w.q_len) if rows is None else np.asarray(rows)
        q = np.ascontiguousarray(H.to_f32_numpy(inp.q[b])[sel][:, hsel])
        pos = (L - w.q_len + np.arange(w.q_len))[sel].astype(np.int32)
        win = int(w.window[b]) if w.window is not None else 0
        snk = int(w.sinks[b]) if (w.sinks is not None and win > 0) else 0
        cap = float(w.softcap[b]) if w.softcap is not None else 0.0
        ro, rl = oracle.attend(q, k, v, pos, hm, w.scale, win, snk, cap, causal=causal,
                               alibi=None if slopes is None else slopes.astype(np.float64),
                               mask=None if mask is None else mask[b][sel][:, :L], allow_empty=True)
        got_o, got_l = out_h[b][sel][:, hsel], lse_h[b][sel][:, hsel]
        empty = np.isneginf(rl)
        assert np.isnan(got_o[empty]).all() and np.isneginf(got_l[empty]).all(), f"{what}: empty rows"
        H.assert_close(got_o[~empty], ro[~empty], w.dtype, f"{what} out[b={b}]")
        H.assert_close(got_l[~empty], rl[~empty], w.dtype, f"{what} lse[b={b}]")


def wl(dtype, hq, hkv, d, page, q_len, lens, seed=41, window=None, sinks=None, softcap=None):
    lens = np.asarray(lens, np.int32)
    w = workloads.Workload("mods_case", seed=seed, batch=len(lens), hq=hq, hkv=hkv, head_dim=d, page_size=page,
                           dtype=dtype, q_len=q_len, context_lens=lens, scale=1.0 / math.sqrt(d),
                           shuffle_pages=True)
    if window is not None:
        w.window = np.asarray(window, np.int32)
        w.sinks = np.asarray(sinks, np.int32)
        w.softcap = np.asarray(softcap, np.float32)
    return w


CASES = [
    # (dtype, hq, hkv, d, page, q_len, lens, causal, alibi, mask density or None)
    ("f32", 8, 2, 64, 16, 1, (300, 77), True, True, 0.7),        # decode-shaped, split path
    ("f32", 8, 2, 64, 16, 16, (256, 40), False, True, None),     # short non-causal suffix
    ("f32", 4, 1, 128, 8, 37, (37, 100), False, False, 0.5),
    ("bf16", 8, 2, 128, 16, 20, (500, 33), False, False, 0.5),
    ("bf16", 4, 4, 64, 32, 1, (1000,), True, True, 0.3),
    ("bf16", 8, 2, 128, 16, 100, (100, 300), False, True, None),  # tiled
    ("bf16", 2, 2, 64, 64, 257, (400, 257), False, False, 0.6),
    ("bf16", 6, 2, 128, 1, 70, (80,), False, True, 0.8),          # tiled, one-token pages
    ("bf16", 16, 1, 64, 64, 96, (200,), True, True, 0.5),
    ("f32", 8, 2, 128, 16, 100, (100, 300), False, True, 0.7),    # fp32 tiled
    ("f32", 4, 1, 64, 32, 70, (500,), True, True, None),
    ("f32", 2, 2, 128, 128, 257, (3000,), False, False, 0.4),
    # ALiBi walks the key blocks outward from the diagonal (here over 3000
    # one-token pages, in key splits of 8 blocks), with and without a listed
    # mask; test_alibi_walk_moves_the_page_window runs unsplit walks that
    # move the page-id window
    ("bf16", 4, 1, 64, 1, 64, (3000,), True, True, None),
    ("bf16", 4, 1, 64, 1, 3000, (3000,), False, True, None),
    ("bf16", 4, 1, 64, 1, 64, (3000,), True, True, 0.9),
    ("bf16", 4, 1, 64, 1, 1000, (3000,), False, True, 0.9),
    ("f32", 4, 1, 64, 1, 64, (3000,), True, True, None),
    ("f32", 4, 1, 64, 1, 3000, (3000,), False, True, None),
    ("f32", 4, 1, 64, 1, 64, (3000,), True, True, 0.9),
    ("f32", 4, 1, 64, 1, 1000, (3000,), False, True, 0.9),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-h{c[1]}x{c[2]}-d{c[3]}-p{c[4]}-q{c[5]}-"
                                                     f"{'c' if c[7] else 'nc'}{'-alibi' if c[8] else ''}"
                                                     f"{'-mask' if c[9] else ''}")
def test_mods_match_oracle(case):
    dtype, hq, hkv, d, page, q_len, lens, causal, alibi, density = case
    say(f"[mods] {case}")
    w = wl(dtype, hq, hkv, d, page, q_len, lens)
    inp = H.build(w, poison=True)
    slopes = alibi_slopes(hq) if alibi else None
    mask = make_mask(w, density, seed=7) if density else None
    out, lse = run_mods(inp, causal, slopes, mask)
    torch.cuda.synchronize()
    check_mods(inp, out, lse, causal, slopes, mask, str(case))


@pytest.mark.parametrize("dtype,q_len", [("bf16", 130), ("f32", 130), ("bf16", 9), ("f32", 1)])
def test_mods_with_window_sinks_softcap(dtype, q_len):
    w = wl(dtype, 8, 2, 128, 32, q_len, (900, 400), window=(200, 64), sinks=(3, 0), softcap=(5.0, 0.0))
    say(f"[mods] window / sinks / softcap + ALiBi + mask, {dtype} q_len={q_len}")
    inp = H.build(w)
    slopes = alibi_slopes(8)
    mask = make_mask(w, 0.8, seed=8)
    out, lse = run_mods(inp, True, slopes, mask)
    torch.cuda.synchronize()
    check_mods(inp, out, lse, True, slopes, mask, f"variants {dtype} {q_len}")


@pytest.mark.parametrize("dtype,q_len", [("bf16", 100), ("f32", 100), ("bf16", 12), ("f32", 12)])
def test_fully_masked_rows_are_nan(dtype, q_len):
    w = wl(dtype, 4, 2, 64, 16, q_len, (150, 120))
    say(f"[mods] fully masked rows, {dtype} q_len={q_len}")
    inp = H.build(w)
    mask = make_mask(w, 0.5, seed=9, empty_rows=5)
    out, lse = run_mods(inp, False, None, mask)
    torch.cuda.synchronize()
    assert torch.isnan(out[0, :5]).all() and torch.isneginf(lse[0, :5]).all()
    check_mods(inp, out, lse, False, None, mask, f"empty rows {dtype}")


@pytest.mark.parametrize("dtype,q_len", [("bf16", 100), ("f32", 100), ("bf16", 10), ("f32", 1)])
def test_no_op_mods_equal_the_plain_call(dtype, q_len):
    """causal = 1 without slopes or mask runs the plain kernels: bit-identical
    to atlas_attend_prefill."""
    import exact_paged_causal_amd as atlas
    w = wl(dtype, 8, 2, 128, 16, q_len, (300, q_len + 5))
    say(f"[mods] no-op mods, {dtype} q_len={q_len}")
    inp = H.build(w)
    o1, l1 = run_mods(inp, True, None, None)
    o1, l1 = o1.clone(), l1.clone()
    o2, l2 = atlas.atlas_attend_prefill(inp.q, inp.k, inp.v, inp.page_table, inp.context_lens, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype,causal", [("bf16", True), ("bf16", False), ("f32", True)])
def test_mods_causal_prefill_full_size(dtype, causal):
    """The causal-prefill shape (S=8192, Hq=32, Hkv=8, D=128; bf16, and fp32
    on the split-operand kernel) with ALiBi slopes, causal and non-causal:
    every row of one seeded q-head per K/V head, and the first and last 512
    rows of every q-head."""
    w = workloads.make("causal_prefill", dtype=dtype)
    say(f"[mods] causal_prefill shape with ALiBi, {dtype} causal={causal}")
    inp = H.build(w)
    slopes = alibi_slopes(w.hq)
    out, lse = run_mods(inp, causal, slopes, None)
    torch.cuda.synchronize()
    for rows, heads in H.full_size_blocks(w, seed=2):
        say(f"[mods] oracle on {len(rows)} rows x heads {heads.tolist()}")
        check_mods(inp, out, lse, causal, slopes, None, f"full size {dtype} causal={causal}", rows=rows, heads=heads)
    assert not torch.isnan(out).any()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_block_sparse_document_mask(dtype):
    """Causal rows inside documents of 150 tokens (block-diagonal mask): the
    bf16 tiled kernel drops the key blocks no row of a query block sees.
    The first 64 query positions of sequence 0 see nothing at all (a whole
    query block with no listed key block): NaN with lse = -inf."""
    w = wl(dtype, 8, 2, 128, 16, 700, (700, 900))
    say(f"[mods] document mask, {dtype}")
    inp = H.build(w, poison=True)
    L = int(inp.layout.page_table.shape[1]) * w.page_size
    mask = np.zeros((w.batch, w.q_len, L), bool)
    j = np.arange(L)
    for b in range(w.batch):
        pos = int(w.context_lens[b]) - w.q_len + np.arange(w.q_len)
        mask[b] = (j[None, :] // 150) == (pos[:, None] // 150)
    mask[0, :64] = False
    out, lse = run_mods(inp, True, None, mask)
    torch.cuda.synchronize()
    assert torch.isnan(out[0, :64]).all() and torch.isneginf(lse[0, :64]).all()
    check_mods(inp, out, lse, True, None, mask, f"document mask {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_document_mask_full_size(dtype):
    """The causal-prefill shape (S=8192, Hq=32, Hkv=8, D=128; bf16, and fp32
    on the split-operand kernel) packed with four documents of 2048 tokens (a
    causal block-diagonal mask, as the benchmark runs it): key blocks inside
    a document are wholly visible to a query block's rows and skip the
    per-score mask.  Every row of one seeded q-head per K/V head, and the
    first and last 512 rows of every q-head."""
    w = workloads.make("causal_prefill", dtype=dtype)
    say(f"[mods] causal_prefill shape with a 4 x 2048 document mask, {dtype}")
    inp = H.build(w)
    L = int(inp.layout.page_table.shape[1]) * w.page_size
    j = np.arange(L)
    pos = np.arange(w.q_len)
    mask = ((j[None, :] // 2048 == pos[:, None] // 2048) & (j[None, :] <= pos[:, None]))[None]
    out, lse = run_mods(inp, True, None, mask)
    torch.cuda.synchronize()
    for rows, heads in H.full_size_blocks(w, seed=3):
        say(f"[mods] oracle on {len(rows)} rows x heads {heads.tolist()}")
        check_mods(inp, out, lse, True, None, mask, f"document mask full size {dtype}", rows=rows, heads=heads)
    assert not torch.isnan(out).any()


def test_mask_past_the_listing_capacity_f32():
    """fp32 tiled prefill with mask bits over more candidate key blocks than a
    workgroup lists (1024 blocks of 64 keys): 8192 queries at the end of a
    67000-token context, one q-head per K/V head (256 positions per
    workgroup, 256 workgroups, no key splits), documents of 20000 tokens with
    causal rows.  The first query blocks list their blocks; the later ones
    compute every candidate block under the per-score mask.  Rows around the
    document boundary and at both ends, every q-head."""
    w = wl("f32", 8, 8, 64, 128, 8192, (67000,), seed=43)
    say("[mods] fp32 mask past the listing capacity: ctx 67000, q_len 8192")
    inp = H.build(w)
    L = int(inp.layout.page_table.shape[1]) * w.page_size
    j = np.arange(L)
    pos = 67000 - w.q_len + np.arange(w.q_len)
    mask = ((j[None, :] // 20000 == pos[:, None] // 20000) & (j[None, :] <= pos[:, None]))[None]
    out, lse = run_mods(inp, True, None, mask)
    torch.cuda.synchronize()
    rows = np.r_[0:40, 60000 - int(pos[0]) - 40:60000 - int(pos[0]) + 40, w.q_len - 60:w.q_len]
    check_mods(inp, out, lse, True, None, mask, "mask past the listing capacity", rows=rows)
    assert not torch.isnan(out).any()


WALK_CASES = [
    # (dtype, q_len, causal, mask): 8192 one-token pages per sequence
    ("bf16", 8192, True, False),
    ("bf16", 4096, False, True),
    ("f32", 8192, True, True),
    ("f32", 4096, False, False),
]


@pytest.mark.parametrize("case", WALK_CASES, ids=lambda c: f"{c[0]}-q{c[1]}-{'c' if c[2] else 'nc'}"
                                                           f"{'-mask' if c[3] else ''}")
def test_alibi_walk_moves_the_page_window(case):
    """ALiBi rows walk their key blocks from the diagonal leftwards (then
    rightwards for non-causal rows).  With one-token pages and one q-head per
    K/V head (256 positions per workgroup, 8 K/V heads, 256 workgroups: no
    key splits), a workgroup's keys span up to 8192 pages, so the page-id
    window (2048 entries bf16, 1024 fp32) moves backwards during the walk
    and forwards again past the diagonal.  With a mask, the listed walk
    skips every block whose keys are hidden from all rows (one block in
    five) and applies the mask bits on the others."""
    dtype, q_len, causal, masked = case
    B = 8192 // q_len
    w = wl(dtype, 8, 8, 64, 1, q_len, (8192,) * B, seed=45)
    # the plan has no key splits: its workspace is the 256-byte header alone
    from exact_paged_causal_amd import atlas as A
    a = A.AttnArgs()
    a.q_dtype = a.kv_dtype = 1 if dtype == "bf16" else 0
    a.batch, a.q_len, a.num_q_heads, a.num_kv_heads, a.head_dim = B, q_len, 8, 8, 64
    a.page_size, a.num_phys_pages, a.max_pages_per_seq, a.scale = 1, 8192 * B, 8192, w.scale
    assert A.atlas_prefill_workspace_bytes(a) == 256
    say(f"[mods] ALiBi walk over 8192 one-token pages, {dtype} q_len={q_len} causal={causal} mask={masked}")
    inp = H.build(w)
    slopes = alibi_slopes(8)
    mask = None
    if masked:
        i = np.arange(q_len)[:, None]
        j = np.arange(8192)[None, :]
        keep = ((j // 64) % 5 != 2) & ((j * 7 + i * 3) % 10 != 0)
        keep |= j == (8192 - q_len + i)
        mask = np.broadcast_to(keep, (B, q_len, 8192))
    out, lse = run_mods(inp, causal, slopes, mask)
    torch.cuda.synchronize()
    rows = np.r_[0:16, q_len // 2 - 8:q_len // 2 + 8, q_len - 48:q_len]
    check_mods(inp, out, lse, causal, slopes, mask, f"walk {case}", rows=rows)
    assert not torch.isnan(out).any()

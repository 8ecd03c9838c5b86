"""CPU tests of the boundary: the library loads and exports every entry point
include/atlas.h declares, host-visible argument errors are reported before any
launch, and the split planner is checked against brute-force enumeration.
No test here launches a kernel."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "atlas.h")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(atlas_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    assert names == sorted(["atlas_abi_version", "atlas_status_str", "atlas_last_error",
                            "atlas_decode_workspace_bytes", "atlas_prefill_workspace_bytes",
                            "atlas_attend_decode", "atlas_attend_prefill", "atlas_attend_mods",
                            "atlas_regenerate_pages", "atlas_attend_decode_regen",
                            "atlas_attend_decode_noalloc", "atlas_append_kv",
                            "atlas_pool_create", "atlas_pool_destroy", "atlas_pool_alloc",
                            "atlas_pool_retain", "atlas_pool_release", "atlas_pool_free_pages",
                            "atlas_pool_refcount", "atlas_cache_create", "atlas_cache_destroy",
                            "atlas_cache_plan", "atlas_cache_drop_sequence", "atlas_cache_get_stats"])


def test_library_exports_every_declared_symbol():
    from exact_paged_causal_amd import atlas as A
    lib = ctypes.CDLL(A.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", A.LIB_PATH], capture_output=True, text=True,
                        check=True).stdout
    exported = set(re.findall(r" T (atlas_\w+)", nm))
    assert exported == set(_declared_functions())
    assert A.atlas_abi_version() == 2
    assert A.atlas_status_str(A.ATLAS_ERR_POOL) == "page id outside the physical pool"


def _struct_offsets_from_header(struct):
    """Field order of a struct in atlas.h (names only)."""
    text = open(HEADER).read()
    body = re.search(r"typedef struct %s \{(.*?)\} %s;" % (struct, struct), text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    return re.findall(r"(\w+)\s*;", body)


def test_binding_structs_mirror_the_header():
    from exact_paged_causal_amd import atlas as A
    assert [f[0] for f in A.AttnArgs._fields_] == _struct_offsets_from_header("atlas_attn_args")
    assert [f[0] for f in A.RegenArgs._fields_] == _struct_offsets_from_header("atlas_regen_args")
    assert [f[0] for f in A.RegenJob._fields_] == _struct_offsets_from_header("atlas_regen_job")
    assert ctypes.sizeof(A.AttnArgs) == 4 * 12 + 8 * 13
    assert A.AttnArgs.head_map.offset == 48
    assert ctypes.sizeof(A.RegenArgs) == 8 + 4 * 8 + 8 * 3
    assert [f[0] for f in A.AttnMods._fields_] == _struct_offsets_from_header("atlas_attn_mods")
    assert ctypes.sizeof(A.AttnMods) == 4 * 2 + 8 * 2
    assert [f[0] for f in A.CacheConfig._fields_] == _struct_offsets_from_header("atlas_cache_config")
    assert [f[0] for f in A.CacheStats._fields_] == _struct_offsets_from_header("atlas_cache_stats")
    assert ctypes.sizeof(A.CacheConfig) == 8 * 2 + 4 * 4 and ctypes.sizeof(A.CacheStats) == 8 * 7


FAKE = 0x10000  # never dereferenced: every case below fails host validation first


def _valid_args(**over):
    from exact_paged_causal_amd import atlas as A
    a = A.AttnArgs()
    a.q_dtype, a.kv_dtype = 0, 0
    a.batch, a.q_len, a.num_q_heads, a.num_kv_heads, a.head_dim = 2, 1, 8, 2, 64
    a.page_size, a.num_phys_pages, a.max_pages_per_seq, a.split_tokens, a.scale = 16, 10, 4, 0, 0.125
    for f in ("q", "k_pages", "v_pages", "page_table", "context_lens", "out", "workspace"):
        setattr(a, f, FAKE)
    a.workspace_bytes = 1 << 40
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("field,value,status", [
    ("q_dtype", 5, 4), ("kv_dtype", 5, 4), ("q_dtype", -1, 4), ("batch", 0, 2), ("q_len", 0, 2), ("q_len", 2, 2),      # decode needs q_len 1
    ("num_q_heads", 7, 2), ("num_kv_heads", 0, 2), ("num_q_heads", 512, 4),
    ("head_dim", 96, 4), ("page_size", 0, 2), ("page_size", 24, 4), ("page_size", 8192, 4),
    ("num_phys_pages", 0, 2), ("max_pages_per_seq", 0, 2), ("split_tokens", -1, 3),
    ("max_pages_per_seq", 1 << 30, 3), ("q", None, 1), ("page_table", None, 1),
    ("out", None, 1), ("workspace_bytes", 16, 5), ("workspace", FAKE + 8, 5), ("scale", float("inf"), 3),
    ("scale", 0.0, 3),
    ("scale", -0.5, 3),
])
def test_decode_rejects_bad_arguments_before_launch(field, value, status):
    from exact_paged_causal_amd import atlas as A
    a = _valid_args(**{field: value})
    st = A.lib.atlas_attend_decode(ctypes.byref(a), None)
    assert st == status, (st, A.atlas_last_error())
    assert A.atlas_last_error() != ""


def test_dtype_pairs():
    """(q_dtype, kv_dtype): (f32, f32), (bf16, bf16) and an fp32 query over a
    bf16 cache have kernels; a bf16 query over an fp32 cache does not."""
    from exact_paged_causal_amd import atlas as A
    for qd, kd, want in ((0, 0, A.ATLAS_ERR_NULL), (1, 1, A.ATLAS_ERR_NULL), (0, 1, A.ATLAS_ERR_NULL),
                         (1, 0, A.ATLAS_ERR_UNSUPPORTED)):
        # q = NULL: a supported pair gets past the dtype check to the pointer check
        a = _valid_args(q_dtype=qd, kv_dtype=kd, q=None)
        for fn in (A.lib.atlas_attend_decode, A.lib.atlas_attend_prefill):
            st = fn(ctypes.byref(a), None)
            assert st == want, (qd, kd, st, A.atlas_last_error())
        if want == A.ATLAS_ERR_UNSUPPORTED:
            assert "kv_dtype" in A.atlas_last_error()
            assert A.lib.atlas_decode_workspace_bytes(ctypes.byref(a)) == ctypes.c_size_t(-1).value
        else:
            assert A.lib.atlas_decode_workspace_bytes(ctypes.byref(a)) not in (0, ctypes.c_size_t(-1).value)
    # the mixed pair always plans the split-KV path, for prefills too: its
    # workspace holds partial states, unlike the tiled bf16 prefill's header
    mixed = _valid_args(q_dtype=0, kv_dtype=1, q_len=64, max_pages_per_seq=8, num_q_heads=8)
    same = _valid_args(q_dtype=1, kv_dtype=1, q_len=64, max_pages_per_seq=8, num_q_heads=8)
    assert A.lib.atlas_prefill_workspace_bytes(ctypes.byref(same)) == 256
    assert A.lib.atlas_prefill_workspace_bytes(ctypes.byref(mixed)) > 256


def test_prefill_limits_and_head_map():
    from exact_paged_causal_amd import atlas as A
    a = _valid_args(q_len=65, max_pages_per_seq=4, page_size=16)   # 65 > 64-token context
    assert A.lib.atlas_attend_prefill(ctypes.byref(a), None) == A.ATLAS_ERR_RANGE
    bad_map = (ctypes.c_int32 * 8)(0, 1, 2, 0, 1, 0, 1, 0)
    a = _valid_args(head_map=ctypes.cast(bad_map, ctypes.POINTER(ctypes.c_int32)))
    assert A.lib.atlas_attend_decode(ctypes.byref(a), None) == A.ATLAS_ERR_SHAPE
    assert "head_map[2]" in A.atlas_last_error()
    # an explicit map lifts the Hq % Hkv requirement
    ok_map = (ctypes.c_int32 * 7)(0, 1, 0, 1, 0, 1, 0)
    a = _valid_args(num_q_heads=7, head_map=ctypes.cast(ok_map, ctypes.POINTER(ctypes.c_int32)))
    assert A.lib.atlas_decode_workspace_bytes(ctypes.byref(a)) not in (0, ctypes.c_size_t(-1).value)


def test_workspace_sizing():
    from exact_paged_causal_amd import atlas as A
    a = _valid_args()
    n = A.lib.atlas_decode_workspace_bytes(ctypes.byref(a))
    # rows (B*Hq) x splits x (D + 2) floats + a 256-byte header
    rows, d = 2 * 8, 64
    assert (n - 256) % (rows * (d + 2) * 4) == 0 and n > 256
    bad = _valid_args(head_dim=80)
    assert A.lib.atlas_decode_workspace_bytes(ctypes.byref(bad)) == ctypes.c_size_t(-1).value


def test_decode_regen_rejects_bad_arguments_before_launch():
    from exact_paged_causal_amd import atlas as A
    fn = A.lib.atlas_attend_decode_regen
    a = _valid_args(q_dtype=1, kv_dtype=0)        # no kernel for a bf16 query over fp32 pages
    assert fn(ctypes.byref(a), 7, 0, None, None) == A.ATLAS_ERR_UNSUPPORTED
    for qd, kd in ((0, 0), (1, 1), (0, 1)):      # every supported pair gets past the dtype check
        a = _valid_args(q_dtype=qd, kv_dtype=kd, q=None)
        assert fn(ctypes.byref(a), 7, 0, None, None) == A.ATLAS_ERR_NULL, (qd, kd)
    for layer in (-1, 1 << 16):
        assert fn(ctypes.byref(_valid_args()), 7, layer, None, None) == A.ATLAS_ERR_RANGE, layer
    assert fn(ctypes.byref(_valid_args(q_len=2)), 7, 0, None, None) == A.ATLAS_ERR_SHAPE   # decode only
    assert fn(ctypes.byref(_valid_args(q=None)), 7, 0, None, None) == A.ATLAS_ERR_NULL
    assert fn(ctypes.byref(_valid_args(workspace_bytes=16)), 7, 0, FAKE, None) == A.ATLAS_ERR_WORKSPACE
    assert A.ATLAS_PAGE_REGENERATE == -1
    assert "#define ATLAS_PAGE_REGENERATE (-1)" in open(HEADER).read()


def test_noalloc_decode_rejects_before_touching_the_gpu():
    """The allocation-free decode checks sizes on the host first: bad shapes
    report the decode's own status; partial states beyond the library's
    32 MiB array are ATLAS_ERR_WORKSPACE, whatever workspace is passed."""
    from exact_paged_causal_amd import atlas as A
    fn = A.lib.atlas_attend_decode_noalloc
    assert fn(None, None) == A.ATLAS_ERR_NULL
    assert fn(ctypes.byref(_valid_args(head_dim=96)), None) == A.ATLAS_ERR_UNSUPPORTED
    assert fn(ctypes.byref(_valid_args(q_len=2)), None) == A.ATLAS_ERR_SHAPE
    # 64 x 64 rows x 16 spans of 4096 keys x 130 floats = 34 MiB > 32 MiB
    big = _valid_args(batch=64, num_q_heads=64, num_kv_heads=8, head_dim=128, page_size=4096,
                      max_pages_per_seq=16, split_tokens=4096)
    need = A.lib.atlas_decode_workspace_bytes(ctypes.byref(big))
    assert need > A.NOALLOC_SCRATCH_BYTES
    assert fn(ctypes.byref(big), None) == A.ATLAS_ERR_WORKSPACE
    assert "32" in A.atlas_last_error() or str(A.NOALLOC_SCRATCH_BYTES) in A.atlas_last_error()
    assert "#define ATLAS_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)" in open(HEADER).read()


def test_mods_reject_bad_arguments_before_launch():
    """atlas_attend_mods: causal must be 0 or 1, windows and sinks need
    causal rows, and a mask row must cover the largest context
    (max_pages_per_seq * page_size = 64 keys -> 2 words)."""
    from exact_paged_causal_amd import atlas as A
    fn = A.lib.atlas_attend_mods
    m = A.AttnMods(2, 0, None, None)
    assert fn(ctypes.byref(_valid_args()), ctypes.byref(m), None) == A.ATLAS_ERR_RANGE
    win = (ctypes.c_int32 * 2)(16, 16)
    a = _valid_args(window=ctypes.addressof(win))
    m = A.AttnMods(0, 0, None, None)
    assert fn(ctypes.byref(a), ctypes.byref(m), None) == A.ATLAS_ERR_UNSUPPORTED
    assert "causal" in A.atlas_last_error()
    m = A.AttnMods(1, 1, None, FAKE)
    assert fn(ctypes.byref(_valid_args()), ctypes.byref(m), None) == A.ATLAS_ERR_SHAPE
    assert "mask_words" in A.atlas_last_error()
    m = A.AttnMods(1, 2, None, FAKE)             # enough words: the call gets past the mods checks
    assert fn(ctypes.byref(_valid_args(q=None)), ctypes.byref(m), None) == A.ATLAS_ERR_NULL


def test_append_rejects_bad_arguments_before_launch():
    from exact_paged_causal_amd import atlas as A
    a = A.AppendArgs()
    a.dtype, a.batch, a.n_new, a.num_kv_heads, a.head_dim = 0, 2, 3, 2, 64
    a.page_size, a.num_phys_pages, a.max_pages_per_seq = 16, 8, 4
    a.k_new = a.v_new = a.page_table = a.start_pos = a.k_pages = a.v_pages = FAKE
    for field, value, status in [("dtype", 3, 4), ("head_dim", 80, 4), ("page_size", 12, 4),
                                 ("batch", 0, 2), ("n_new", -1, 2), ("num_phys_pages", 0, 2),
                                 ("max_pages_per_seq", 0, 2), ("k_new", None, 1), ("start_pos", None, 1)]:
        saved = getattr(a, field)
        setattr(a, field, value)
        assert A.lib.atlas_append_kv(ctypes.byref(a), None) == status, field
        setattr(a, field, saved)
    a.n_new = 0   # nothing to write is not an error (and touches nothing)
    a.k_new = None
    assert A.lib.atlas_append_kv(ctypes.byref(a), None) == A.ATLAS_OK
    assert ctypes.sizeof(A.AppendArgs) == 4 * 8 + 8 * 6
    assert [f[0] for f in A.AppendArgs._fields_] == _struct_offsets_from_header("atlas_append_args")


def test_page_pool_bookkeeping():
    """Allocation order, all-or-nothing exhaustion, shared pages kept until the
    last release, and errors that change nothing."""
    from exact_paged_causal_amd import atlas as A
    pool = A.PagePool(6)
    assert pool.free_pages() == 6
    a = pool.alloc(4)
    assert a == [0, 1, 2, 3] and pool.free_pages() == 2
    with pytest.raises(A.AtlasError) as ei:
        pool.alloc(3)                                    # only 2 free: nothing handed out
    assert ei.value.status == A.ATLAS_ERR_POOL and pool.free_pages() == 2
    pool.retain([0, 1])                                  # a second sequence shares the prefix pages
    assert [pool.refcount(i) for i in range(6)] == [2, 2, 1, 1, 0, 0]
    pool.release([0, 1, 2, 3])                           # first sequence ends
    assert [pool.refcount(i) for i in range(6)] == [1, 1, 0, 0, 0, 0] and pool.free_pages() == 4
    with pytest.raises(A.AtlasError) as ei:
        pool.release([0, 0])                             # would drop below zero: no change
    assert ei.value.status == A.ATLAS_ERR_RANGE and pool.refcount(0) == 1
    for bad in ([2], [7], [-1]):                         # free, outside, negative
        with pytest.raises(A.AtlasError):
            pool.retain(bad)
    with pytest.raises(A.AtlasError):
        pool.release([6])
    pool.release([1, 0])
    assert pool.free_pages() == 6 and pool.refcount(6) == -1
    assert sorted(pool.alloc(6)) == list(range(6)) and pool.free_pages() == 0
    assert pool.alloc(0) == []
    pool.close()
    h = ctypes.c_void_p()
    assert A.lib.atlas_pool_create(0, ctypes.byref(h)) == A.ATLAS_ERR_SHAPE


def test_regenerate_rejects_bad_arguments():
    from exact_paged_causal_amd import atlas as A
    r = A.RegenArgs()
    r.dtype, r.num_kv_heads, r.head_dim, r.page_size, r.num_phys_pages, r.num_jobs = 0, 2, 64, 16, 4, 1
    r.jobs = r.k_pages = r.v_pages = FAKE
    for field, value, status in [("head_dim", 32, 4), ("page_size", 3, 4), ("layer", 1 << 16, 3),
                                 ("num_jobs", -1, 2), ("dtype", 9, 4)]:
        saved = getattr(r, field)
        setattr(r, field, value)
        assert A.lib.atlas_regenerate_pages(ctypes.byref(r), None) == status, field
        setattr(r, field, saved)
    r.jobs = None
    assert A.lib.atlas_regenerate_pages(ctypes.byref(r), None) == A.ATLAS_ERR_NULL
    r.num_jobs = 0   # nothing to do is not an error
    assert A.lib.atlas_regenerate_pages(ctypes.byref(r), None) == A.ATLAS_OK


# ---------------------------------------------------------------- planner

@pytest.fixture(scope="module")
def planner(tmp_path_factory):
    so = str(tmp_path_factory.mktemp("plan") / "plan_probe.so")
    subprocess.run(["g++", "-O1", "-std=c++17", "-fPIC", "-shared",
                    "-I", os.path.join(ROOT, "exact_paged_causal_amd", "csrc"),
                    os.path.join(ROOT, "tests", "plan_probe.cpp"), "-o", so], check=True)
    lib = ctypes.CDLL(so)
    ip = ctypes.POINTER(ctypes.c_int)
    lib.probe_plan.argtypes = [ctypes.c_int] * 5 + [ip]
    lib.probe_ranges.argtypes = [ctypes.c_int] * 5 + [ip, ctypes.c_int, ip]
    lib.probe_bound.argtypes = [ctypes.c_int] * 3
    lib.probe_chunk.argtypes = [ctypes.c_int] * 5 + [ip]
    lib.probe_tiled.argtypes = [ctypes.c_int] * 5 + [ip, ctypes.c_int, ip]
    return lib


def _ranges(lib, pmin, pmax, w, s, t):
    buf = (ctypes.c_int * 4096)()
    n = ctypes.c_int()
    lib.probe_ranges(pmin, pmax, w, s, t, buf, 2048, ctypes.byref(n))
    return [(buf[2 * i], buf[2 * i + 1]) for i in range(n.value)]


def _union_visible(pmin, pmax, w, s):
    keys = set()
    for pos in range(max(pmin, 0), pmax + 1):
        if w <= 0:
            keys |= set(range(pos + 1))
        else:
            keys |= set(range(max(0, pos - w + 1), pos + 1)) | set(range(min(s, pos + 1)))
    return keys


def test_split_ranges_cover_exactly_the_visible_keys(planner):
    """Splits are disjoint, ordered, at most T keys each, cut at multiples of
    T, cover exactly the union of the rows' visible keys, and never exceed
    the host's bound."""
    rng = np.random.default_rng(0)
    for _ in range(1500):
        ctx = int(rng.integers(1, 400))
        q_len = int(rng.integers(1, min(ctx, 40) + 1))
        pmin = ctx - q_len + int(rng.integers(0, q_len))
        pmax = int(rng.integers(pmin, ctx))
        w = int(rng.choice([0, 1, 2, 5, 17, 64, 1000]))
        s = int(rng.choice([0, 1, 4, 30, 500]))
        t = int(rng.choice([1, 3, 16, 64, 128]))
        rs = _ranges(planner, pmin, pmax, w, s, t)
        keys = []
        for a, b in rs:
            assert 0 <= a < b <= pmax + 1 and b - a <= t
            assert a // t == (b - 1) // t, "split crosses a T boundary"
            keys.extend(range(a, b))
        assert keys == sorted(keys) and len(keys) == len(set(keys))
        assert set(keys) == _union_visible(pmin, pmax, w, s), (pmin, pmax, w, s, t)
        max_ctx = ctx + int(rng.integers(0, 50))
        assert len(rs) <= planner.probe_bound(max_ctx, t, 1 if (w > 0 and s > 0) else 0)


def test_split_plan_edge_cases(planner):
    out = (ctypes.c_int * 6)()
    planner.probe_plan(-1, -1, 0, 0, 64, out)          # no valid row
    assert out[0] == 0
    assert _ranges(planner, 0, 0, 0, 0, 64) == [(0, 1)]          # one-token history
    assert _ranges(planner, 99, 99, 1, 0, 64) == [(99, 100)]     # window of one
    assert _ranges(planner, 99, 99, 1, 4, 64) == [(0, 4), (99, 100)]
    assert _ranges(planner, 99, 99, 10, 200, 64) == [(0, 64), (64, 90), (90, 100)]  # sinks reach the window
    assert _ranges(planner, 4095, 4095, 0, 0, 1024) == [(0, 1024), (1024, 2048), (2048, 3072), (3072, 4096)]


def test_chunk_rows(planner):
    out = (ctypes.c_int * 4)()
    # 16 queries x group 4 = 64 rows, 8 per chunk; chunk 3 = rows 24..31 = queries 6, 7
    planner.probe_chunk(3, 8, 4, 16, 256, out)
    assert list(out) == [24, 32, 256 - 16 + 6, 256 - 16 + 7]
    planner.probe_chunk(8, 8, 4, 16, 256, out)   # past the end
    assert out[0] >= out[1]
    planner.probe_chunk(0, 4, 3, 1, 10, out)     # decode, group of 3 in a chunk of 4
    assert list(out) == [0, 3, 9, 9]


@pytest.mark.parametrize("pos_lo,pos_hi,w,s", [
    (0, 0, 0, 0), (0, 63, 0, 0), (100, 163, 0, 0), (5000, 5063, 0, 0), (5000, 5063, 128, 0),
    (5000, 5063, 128, 4), (5000, 5063, 1, 70), (300, 363, 4096, 4), (1000, 1003, 64, 64), (200, 263, 100, 200),
])
def test_tiled_block_list_is_the_visible_blocks(planner, pos_lo, pos_hi, w, s):
    """The key blocks a tiled query block visits (also the merge's split
    count of the tiled key splits) are exactly, in increasing order, the
    64-key blocks holding a key some row at positions [pos_lo, pos_hi] sees."""
    buf = (ctypes.c_int * 4096)()
    n = ctypes.c_int()
    planner.probe_tiled(pos_lo, pos_hi, w, s if w > 0 else 0, 64, buf, 4096, ctypes.byref(n))
    got = list(buf[:n.value])
    want = sorted({k // 64 for k in _union_visible(pos_lo, pos_hi, w, s if w > 0 else 0)})
    assert got == want



def test_short_contexts_plan_one_split_per_row():
    """Contexts up to 256 keys without a sink array plan one split per row
    (the fold writes the rows and no merge runs): the workspace holds one
    partial state per row.  257 keys, or a sink array, plan several."""
    from exact_paged_causal_amd import atlas as A
    sinks = (ctypes.c_int32 * 2)(0, 0)
    win = (ctypes.c_int32 * 2)(8, 8)
    for q_len, fn in ((1, A.lib.atlas_decode_workspace_bytes), (16, A.lib.atlas_prefill_workspace_bytes)):
        rows = 2 * q_len * 8
        per_split = rows * (64 + 2) * 4
        for ctx, page, extra, splits in ((256, 16, {}, 1), (64, 64, {}, 1), (256, 1, {}, 1),
                                         (256, 16, {"window": ctypes.addressof(win)}, 1),
                                         (272, 16, {}, None), (256, 16, {"window": ctypes.addressof(win),
                                                                         "sink_tokens": ctypes.addressof(sinks)}, None)):
            a = _valid_args(q_len=q_len, page_size=page, max_pages_per_seq=ctx // page, num_phys_pages=4096, **extra)
            n = fn(ctypes.byref(a))
            if splits == 1:
                assert n == 256 + per_split, (q_len, ctx, page, extra, n)
            else:
                assert n >= 256 + 2 * per_split, (q_len, ctx, page, extra, n)


def test_split_plan_depends_on_the_cache_dtype():
    """Default splits, never shorter than 128 keys nor (for calls with at
    least 16 work items per split) more than 32 per row.  The matrix-core fold (bf16 cache, also under an fp32 query) aims at two
    work items per CU from 4096 keys; the vector fold (fp32 cache) keeps the
    plan for eight per CU when its splits come out 1024 keys or longer, and
    otherwise aims at two per CU from 512 keys.  8 x 32 q-heads over 8 K/V
    heads at 65536 keys: fp32 32 splits of 2048, bf16 16 of 4096; 4 x 32
    q-heads at 8192 keys: 16 splits of 512 for either.  The plan is the same
    for the decode that generates cold pages, so one workspace serves both."""
    from exact_paged_causal_amd import atlas as A
    for batch, d, pages, cases in ((8, 64, 128, ((0, 0, 32), (1, 1, 16), (0, 1, 16))),
                                   (4, 128, 512, ((0, 0, 16), (1, 1, 16), (0, 1, 16)))):
        rows = batch * 32
        for q_dt, kv_dt, splits in cases:
            a = _valid_args(q_dtype=q_dt, kv_dtype=kv_dt, batch=batch, num_q_heads=32, num_kv_heads=8, head_dim=d,
                            page_size=512 if pages == 128 else 16, max_pages_per_seq=pages, num_phys_pages=1 << 16)
            assert A.lib.atlas_decode_workspace_bytes(ctypes.byref(a)) == 256 + rows * splits * (d + 2) * 4, \
                (batch, q_dt, kv_dt)


def test_few_item_calls_take_more_splits_per_row():
    """A call with few (sequence, K/V head, row chunk) items per split may
    exceed 32 splits per row, up to what two work items per CU (512) need:
    one sequence of 8 fp32 q-heads over one K/V head at 131072 keys takes
    512 splits of 256 keys; a bf16 single head the same; two bf16 sequences
    at 32768 keys 256 splits of 128; with 16 items per split (2 sequences x
    8 K/V heads) the cap stays 32."""
    from exact_paged_causal_amd import atlas as A
    for q_dt, kv_dt, batch, hq, hkv, d, pages, splits in ((0, 0, 1, 8, 1, 128, 1024, 512),
                                                         (1, 1, 1, 1, 1, 128, 1024, 512),
                                                         (1, 1, 2, 1, 1, 64, 256, 256),
                                                         (1, 1, 2, 8, 8, 128, 1024, 32)):
        a = _valid_args(q_dtype=q_dt, kv_dtype=kv_dt, batch=batch, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                        page_size=128, max_pages_per_seq=pages, num_phys_pages=1 << 16)
        rows = batch * hq
        assert A.lib.atlas_decode_workspace_bytes(ctypes.byref(a)) == 256 + rows * splits * (d + 2) * 4, \
            (q_dt, batch, hq, hkv, pages)


def test_prepare_attend_rejects_bad_arguments_before_touching_tensors():
    """prepare_attend: an unknown kind or a missing out tensor is refused
    first (ValueError), before any tensor is inspected."""
    import pytest as _pt
    from exact_paged_causal_amd import atlas as A
    with _pt.raises(ValueError, match="kind"):
        A.prepare_attend("bogus", None, None, None, None, None, 0.1, out=None)
    with _pt.raises(ValueError, match="out"):
        A.prepare_attend("decode", None, None, None, None, None, 0.1, out=None)

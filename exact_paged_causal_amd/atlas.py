"""ctypes binding of libatlas (include/atlas.h), with the same entry-point names.

Argument marshalling only: tensors are checked for device, dtype, layout and
shape, their sizes are filled into the C argument structs, and the call runs
on torch's current HIP stream.  Every step of the computation runs in the HIP
kernels of libatlas.so; if the library is missing, importing this module
raises -- there is no other implementation behind these names.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libatlas.so")

ATLAS_OK = 0
ATLAS_ERR_NULL = 1
ATLAS_ERR_SHAPE = 2
ATLAS_ERR_RANGE = 3
ATLAS_ERR_UNSUPPORTED = 4
ATLAS_ERR_WORKSPACE = 5
ATLAS_ERR_POOL = 6
ATLAS_ERR_NONFINITE = 7
ATLAS_ERR_DEVICE = 8

ATLAS_DTYPE_F32 = 0
ATLAS_DTYPE_BF16 = 1

ATLAS_PAGE_REGENERATE = -1   # page-table value of a page regenerated inside atlas_attend_decode_regen

ABI_VERSION = 2

_DTYPES = {torch.float32: ATLAS_DTYPE_F32, torch.bfloat16: ATLAS_DTYPE_BF16}


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_phys_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("split_tokens", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("head_map", ctypes.POINTER(ctypes.c_int32)),
        ("q", ctypes.c_void_p),
        ("k_pages", ctypes.c_void_p),
        ("v_pages", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("context_lens", ctypes.c_void_p),
        ("window", ctypes.c_void_p),
        ("sink_tokens", ctypes.c_void_p),
        ("softcap", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class RegenJob(ctypes.Structure):
    _fields_ = [("seq", ctypes.c_int32), ("logical_page", ctypes.c_int32),
                ("phys_page", ctypes.c_int32)]


class RegenArgs(ctypes.Structure):
    _fields_ = [
        ("seed", ctypes.c_uint64),
        ("layer", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_phys_pages", ctypes.c_int32),
        ("num_jobs", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
        ("jobs", ctypes.c_void_p),
        ("k_pages", ctypes.c_void_p),
        ("v_pages", ctypes.c_void_p),
    ]


class AppendArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("n_new", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_phys_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("k_new", ctypes.c_void_p),
        ("v_new", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("start_pos", ctypes.c_void_p),
        ("k_pages", ctypes.c_void_p),
        ("v_pages", ctypes.c_void_p),
    ]


class AttnMods(ctypes.Structure):
    """atlas_attn_mods: causal flag, mask row length, ALiBi slopes, mask bits."""
    _fields_ = [
        ("causal", ctypes.c_int32),
        ("mask_words", ctypes.c_int32),
        ("alibi_slopes", ctypes.c_void_p),
        ("mask_bits", ctypes.c_void_p),
    ]


class CacheConfig(ctypes.Structure):
    """atlas_cache_config."""
    _fields_ = [
        ("hot_cache_bytes", ctypes.c_int64),
        ("page_bytes", ctypes.c_int64),
        ("page_size", ctypes.c_int32),
        ("recent_tokens", ctypes.c_int32),
        ("admit_regenerated", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class CacheStats(ctypes.Structure):
    """atlas_cache_stats."""
    _fields_ = [(n, ctypes.c_int64) for n in ("capacity_pages", "resident_pages", "resident_bytes", "hits",
                                              "misses", "admitted", "evicted")]


EXPORTS = ("atlas_abi_version", "atlas_status_str", "atlas_last_error",
           "atlas_decode_workspace_bytes", "atlas_prefill_workspace_bytes",
           "atlas_attend_decode", "atlas_attend_prefill", "atlas_attend_mods", "atlas_regenerate_pages",
           "atlas_attend_decode_regen", "atlas_attend_decode_noalloc", "atlas_append_kv", "atlas_pool_create", "atlas_pool_destroy",
           "atlas_pool_alloc", "atlas_pool_retain", "atlas_pool_release", "atlas_pool_free_pages",
           "atlas_pool_refcount", "atlas_cache_create", "atlas_cache_destroy", "atlas_cache_plan",
           "atlas_cache_drop_sequence", "atlas_cache_get_stats")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libatlas.so is not built ({LIB_PATH}); run __graft_entry__.build() "
                          "or python exact_paged_causal_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    lib.atlas_abi_version.restype = ctypes.c_int32
    lib.atlas_abi_version.argtypes = []
    lib.atlas_status_str.restype = ctypes.c_char_p
    lib.atlas_status_str.argtypes = [ctypes.c_int32]
    lib.atlas_last_error.restype = ctypes.c_char_p
    lib.atlas_last_error.argtypes = []
    for name in ("atlas_decode_workspace_bytes", "atlas_prefill_workspace_bytes"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_size_t
        fn.argtypes = [ctypes.POINTER(AttnArgs)]
    for name in ("atlas_attend_decode", "atlas_attend_prefill"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int32
        fn.argtypes = [ctypes.POINTER(AttnArgs), ctypes.c_void_p]
    lib.atlas_attend_mods.restype = ctypes.c_int32
    lib.atlas_attend_mods.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(AttnMods), ctypes.c_void_p]
    lib.atlas_regenerate_pages.restype = ctypes.c_int32
    lib.atlas_regenerate_pages.argtypes = [ctypes.POINTER(RegenArgs), ctypes.c_void_p]
    lib.atlas_attend_decode_regen.restype = ctypes.c_int32
    lib.atlas_attend_decode_regen.argtypes = [ctypes.POINTER(AttnArgs), ctypes.c_uint64, ctypes.c_int32,
                                              ctypes.c_void_p, ctypes.c_void_p]
    lib.atlas_attend_decode_noalloc.restype = ctypes.c_int32
    lib.atlas_attend_decode_noalloc.argtypes = [ctypes.POINTER(AttnArgs), ctypes.c_void_p]
    lib.atlas_append_kv.restype = ctypes.c_int32
    lib.atlas_append_kv.argtypes = [ctypes.POINTER(AppendArgs), ctypes.c_void_p]
    lib.atlas_pool_create.restype = ctypes.c_int32
    lib.atlas_pool_create.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p)]
    lib.atlas_pool_destroy.restype = None
    lib.atlas_pool_destroy.argtypes = [ctypes.c_void_p]
    for name in ("atlas_pool_alloc", "atlas_pool_retain", "atlas_pool_release"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int32
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
    lib.atlas_pool_free_pages.restype = ctypes.c_int32
    lib.atlas_pool_free_pages.argtypes = [ctypes.c_void_p]
    lib.atlas_pool_refcount.restype = ctypes.c_int32
    lib.atlas_pool_refcount.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    lib.atlas_cache_create.restype = ctypes.c_int32
    lib.atlas_cache_create.argtypes = [ctypes.POINTER(CacheConfig), ctypes.POINTER(ctypes.c_void_p)]
    lib.atlas_cache_destroy.restype = None
    lib.atlas_cache_destroy.argtypes = [ctypes.c_void_p]
    i32p, i64p = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    lib.atlas_cache_plan.restype = ctypes.c_int32
    lib.atlas_cache_plan.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, i64p, i32p, ctypes.c_int32,
                                     i32p, i32p, ctypes.c_int32, i32p, i32p]
    lib.atlas_cache_drop_sequence.restype = ctypes.c_int32
    lib.atlas_cache_drop_sequence.argtypes = [ctypes.c_void_p, ctypes.c_int64]
    lib.atlas_cache_get_stats.restype = ctypes.c_int32
    lib.atlas_cache_get_stats.argtypes = [ctypes.c_void_p, ctypes.POINTER(CacheStats)]
    if lib.atlas_abi_version() != ABI_VERSION:
        raise ImportError(f"libatlas ABI {lib.atlas_abi_version()} != binding ABI {ABI_VERSION}")
    return lib


lib = _load()


class AtlasError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = lib.atlas_last_error().decode()
        super().__init__(f"{where}: {lib.atlas_status_str(status).decode()} ({status}): {detail}")


def atlas_abi_version() -> int:
    return int(lib.atlas_abi_version())


def atlas_status_str(status: int) -> str:
    return lib.atlas_status_str(status).decode()


def atlas_last_error() -> str:
    return lib.atlas_last_error().decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _current_stream_handle(device_index):
    """Handle of torch's current stream on a device (the raw handle, without
    building a Stream object, where torch offers it)."""
    if _raw_stream is not None:
        return _raw_stream(device_index)
    return torch.cuda.current_stream(device_index).cuda_stream


def _stream(stream, device):
    """The stream argument of a call on `device`: the given stream, else
    torch's current stream of that device."""
    if stream is None:
        return ctypes.c_void_p(_current_stream_handle(device.index))
    return ctypes.c_void_p(stream.cuda_stream)


def _check(t, name, dtype=None, device=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if device is not None and t.get_device() != device.index:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def make_attn_args(q, k_pages, v_pages, page_table, context_lens, scale, *, head_map=None,
                   window=None, sink_tokens=None, softcap=None, out=None, lse=None,
                   workspace=None, split_tokens=0):
    """Fill an AttnArgs from tensors (q [B][q_len][Hq][D], arenas
    [num_phys][Hkv][P][D], page_table [B][max_pages] int32, context_lens [B]
    int32).  q and the arenas may differ in dtype (the library accepts an
    fp32 query over a bf16 cache).  Returns (args, keepalive)."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"q dtype {q.dtype} unsupported (float32 or bfloat16)")
    if k_pages.dtype not in _DTYPES:
        raise ValueError(f"k_pages dtype {k_pages.dtype} unsupported (float32 or bfloat16)")
    dev = q.device
    _check(q, "q", ndim=4)
    _check(k_pages, "k_pages", None, dev, 4)
    _check(v_pages, "v_pages", k_pages.dtype, dev, 4)
    _check(page_table, "page_table", torch.int32, dev, 2)
    _check(context_lens, "context_lens", torch.int32, dev, 1)
    B, q_len, hq, d = q.shape
    num_phys, hkv, P, dk = k_pages.shape
    if v_pages.shape != k_pages.shape or dk != d:
        raise ValueError("k_pages/v_pages shapes must match [num_phys][Hkv][P][D] with q's D")
    if page_table.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("page_table and context_lens need one row per sequence")
    for name, t, dt in (("window", window, torch.int32), ("sink_tokens", sink_tokens, torch.int32),
                        ("softcap", softcap, torch.float32)):
        if t is not None:
            _check(t, name, dt, dev, 1)
            if t.shape[0] != B:
                raise ValueError(f"{name} needs one entry per sequence")
    if out is not None:
        _check(out, "out", torch.float32, dev, 4)
        if tuple(out.shape) != (B, q_len, hq, d):
            raise ValueError("out must be [B][q_len][Hq][D] float32")
    if lse is not None:
        _check(lse, "lse", torch.float32, dev, 3)
        if tuple(lse.shape) != (B, q_len, hq):
            raise ValueError("lse must be [B][q_len][Hq] float32")
    keep = []
    hm_ptr = None
    if head_map is not None:
        hm = (ctypes.c_int32 * hq)(*[int(x) for x in head_map])
        if len(head_map) != hq:
            raise ValueError("head_map needs one entry per q-head")
        keep.append(hm)
        hm_ptr = ctypes.cast(hm, ctypes.POINTER(ctypes.c_int32))
    a = AttnArgs()
    a.q_dtype = _DTYPES[q.dtype]
    a.kv_dtype = _DTYPES[k_pages.dtype]
    a.batch, a.q_len, a.num_q_heads, a.num_kv_heads, a.head_dim = B, q_len, hq, hkv, d
    a.page_size, a.num_phys_pages, a.max_pages_per_seq = P, num_phys, page_table.shape[1]
    a.split_tokens = int(split_tokens)
    a.scale = float(scale)
    a.head_map = hm_ptr
    a.q, a.k_pages, a.v_pages = _ptr(q), _ptr(k_pages), _ptr(v_pages)
    a.page_table, a.context_lens = _ptr(page_table), _ptr(context_lens)
    a.window, a.sink_tokens, a.softcap = _ptr(window), _ptr(sink_tokens), _ptr(softcap)
    a.out, a.lse = _ptr(out), _ptr(lse)
    if workspace is not None:
        _check(workspace, "workspace", None, dev)
        a.workspace = _ptr(workspace)
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    return a, keep


def atlas_decode_workspace_bytes(args: AttnArgs) -> int:
    n = lib.atlas_decode_workspace_bytes(ctypes.byref(args))
    if n == ctypes.c_size_t(-1).value:
        raise AtlasError(lib_status_from_error(), "atlas_decode_workspace_bytes")
    return int(n)


def atlas_prefill_workspace_bytes(args: AttnArgs) -> int:
    n = lib.atlas_prefill_workspace_bytes(ctypes.byref(args))
    if n == ctypes.c_size_t(-1).value:
        raise AtlasError(lib_status_from_error(), "atlas_prefill_workspace_bytes")
    return int(n)


def lib_status_from_error() -> int:
    """Sizing calls report invalid arguments through SIZE_MAX; the status code
    itself is not returned, so report it as a shape/range problem."""
    return ATLAS_ERR_SHAPE


def _attend(entry, ws_fn, q, k_pages, v_pages, page_table, context_lens, scale, out, lse,
            workspace, stream, extra=(), **kw):
    B, q_len, hq, d = q.shape
    want_lse = kw.pop("want_lse", True)
    # Buffers the binding allocates belong to the stream the call runs on:
    # torch's caching allocator may hand a freed block to the next allocation
    # of the stream it was allocated on, so a workspace allocated on another
    # stream could be reused while the kernels still use it.  Without a
    # stream argument the call runs on torch's current stream of q's device,
    # where torch.empty allocates anyway.
    if not q.is_cuda:
        raise ValueError("q must be on the GPU")
    dev = q.device
    if stream is None:
        handle = _current_stream_handle(dev.index)
        alloc = contextlib.nullcontext()   # torch.empty on dev uses dev's current stream
    else:
        handle = stream.cuda_stream
        alloc = torch.cuda.stream(stream)
    need_ws = workspace is None
    with alloc:
        if out is None:
            out = torch.empty((B, q_len, hq, d), dtype=torch.float32, device=dev)
        if lse is None and want_lse:
            lse = torch.empty((B, q_len, hq), dtype=torch.float32, device=dev)
        args, keep = make_attn_args(q, k_pages, v_pages, page_table, context_lens, scale, out=out,
                                    lse=lse, **kw)
        if need_ws:
            workspace = torch.empty(max(ws_fn(args), 1), dtype=torch.uint8, device=dev)
    if need_ws:
        args.workspace = _ptr(workspace)
        args.workspace_bytes = workspace.numel()
    else:
        _check(workspace, "workspace", None, dev)
        args.workspace = _ptr(workspace)
        args.workspace_bytes = workspace.numel() * workspace.element_size()
    st = getattr(lib, entry)(ctypes.byref(args), *extra, ctypes.c_void_p(handle))
    if st != ATLAS_OK:
        raise AtlasError(st, entry)
    return out, lse


def atlas_attend_decode(q, k_pages, v_pages, page_table, context_lens, scale, *, head_map=None,
                        window=None, sink_tokens=None, softcap=None, out=None, lse=None,
                        workspace=None, split_tokens=0, stream=None, want_lse=True):
    """Decode attention (q_len == 1).  Returns (out [B][1][Hq][D] f32, lse [B][1][Hq] f32)."""
    return _attend("atlas_attend_decode", atlas_decode_workspace_bytes, q, k_pages, v_pages,
                   page_table, context_lens, scale, out, lse, workspace, stream,
                   head_map=head_map, window=window, sink_tokens=sink_tokens, softcap=softcap,
                   split_tokens=split_tokens, want_lse=want_lse)


def atlas_attend_decode_regen(q, k_pages, v_pages, page_table, context_lens, scale, seed: int, layer: int = 0,
                              *, seq_keys=None, head_map=None, window=None, sink_tokens=None, softcap=None,
                              out=None, lse=None, workspace=None, split_tokens=0, stream=None, want_lse=True):
    """Decode attention in which page_table entries equal to ATLAS_PAGE_REGENERATE (-1) are
    regenerated inside the kernel from (seed, layer, sequence key, logical page) -- the rows
    atlas_regenerate_pages would write for that key -- instead of read from the arenas.
    seq_keys: int32 [B] device tensor of generator keys in [0, 65536) (None: the batch row).
    Returns (out [B][1][Hq][D] f32, lse [B][1][Hq] f32)."""
    if seq_keys is not None:
        _check(seq_keys, "seq_keys", torch.int32, q.device, 1)
        if seq_keys.shape[0] != q.shape[0]:
            raise ValueError("seq_keys needs one entry per sequence")
    return _attend("atlas_attend_decode_regen", atlas_decode_workspace_bytes, q, k_pages, v_pages,
                   page_table, context_lens, scale, out, lse, workspace, stream,
                   extra=(ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF), ctypes.c_int32(int(layer)),
                          _ptr(seq_keys)),
                   head_map=head_map, window=window, sink_tokens=sink_tokens, softcap=softcap,
                   split_tokens=split_tokens, want_lse=want_lse)


NOALLOC_SCRATCH_BYTES = 32 << 20   # ATLAS_NOALLOC_SCRATCH_BYTES


def atlas_attend_decode_noalloc(q, k_pages, v_pages, page_table, context_lens, scale, *, out, lse=None,
                                head_map=None, window=None, sink_tokens=None, softcap=None, split_tokens=0,
                                stream=None):
    """atlas_attend_decode whose partial states live in the library's own device array: the
    caller passes the outputs (out [B][1][Hq][D] f32, optionally lse [B][1][Hq] f32) and
    nothing is allocated.  Calls overlapping on one GPU race (one shared array per GPU)."""
    args, keep = make_attn_args(q, k_pages, v_pages, page_table, context_lens, scale, head_map=head_map,
                                window=window, sink_tokens=sink_tokens, softcap=softcap, out=out, lse=lse,
                                split_tokens=split_tokens)
    st = lib.atlas_attend_decode_noalloc(ctypes.byref(args), _stream(stream, q.device))
    if st != ATLAS_OK:
        raise AtlasError(st, "atlas_attend_decode_noalloc")
    return out, lse


def atlas_attend_prefill(q, k_pages, v_pages, page_table, context_lens, scale, *, head_map=None,
                         window=None, sink_tokens=None, softcap=None, out=None, lse=None,
                         workspace=None, split_tokens=0, stream=None, want_lse=True):
    """Suffix-query attention (q_len >= 1).  Returns (out [B][q_len][Hq][D] f32, lse [B][q_len][Hq] f32)."""
    return _attend("atlas_attend_prefill", atlas_prefill_workspace_bytes, q, k_pages, v_pages,
                   page_table, context_lens, scale, out, lse, workspace, stream,
                   head_map=head_map, window=window, sink_tokens=sink_tokens, softcap=softcap,
                   split_tokens=split_tokens, want_lse=want_lse)


def atlas_attend_mods(q, k_pages, v_pages, page_table, context_lens, scale, *, causal: bool = True,
                      alibi_slopes=None, mask_bits=None, head_map=None, window=None, sink_tokens=None,
                      softcap=None, out=None, lse=None, workspace=None, split_tokens=0, stream=None,
                      want_lse=True):
    """atlas_attend_prefill with modifications: causal=False lets every row see the whole
    context; alibi_slopes (f32 [Hq] device tensor) adds -slope * |pos - j| to each logit;
    mask_bits (int32/uint32 [B][q_len][words] device tensor, bit j & 31 of word j >> 5 = key j
    visible) hides keys.  Rows with no visible key come back NaN with lse -inf.
    Returns (out [B][q_len][Hq][D] f32, lse [B][q_len][Hq] f32)."""
    mods = AttnMods()
    mods.causal = 1 if causal else 0
    keep = []
    if alibi_slopes is not None:
        _check(alibi_slopes, "alibi_slopes", torch.float32, q.device, 1)
        if alibi_slopes.shape[0] != q.shape[2]:
            raise ValueError("alibi_slopes needs one slope per q-head")
        mods.alibi_slopes = _ptr(alibi_slopes)
        keep.append(alibi_slopes)
    if mask_bits is not None:
        if mask_bits.dtype not in (torch.int32, torch.uint32) or mask_bits.device != q.device or \
                mask_bits.dim() != 3 or not mask_bits.is_contiguous():
            raise ValueError("mask_bits must be a contiguous 32-bit [B][q_len][words] tensor on q's device")
        if tuple(mask_bits.shape[:2]) != tuple(q.shape[:2]):
            raise ValueError("mask_bits must be [B][q_len][words]")
        mods.mask_bits = _ptr(mask_bits)
        mods.mask_words = mask_bits.shape[2]
        keep.append(mask_bits)
    return _attend("atlas_attend_mods", atlas_prefill_workspace_bytes, q, k_pages, v_pages,
                   page_table, context_lens, scale, out, lse, workspace, stream,
                   extra=(ctypes.byref(mods),), head_map=head_map, window=window, sink_tokens=sink_tokens,
                   softcap=softcap, split_tokens=split_tokens, want_lse=want_lse)


class PreparedAttend:
    """One attention call with fixed tensors, checked and marshalled once.

    Calling it issues the C-ABI call again with the same arguments: the
    tensors' contents (queries, cache pages, page table, lengths, variant
    arrays) may change between calls, their shapes, dtypes and storage may
    not, and the object keeps them alive.  Runs on the given stream, else on
    torch's current stream of the tensors' device at each call.  Returns
    (out, lse)."""

    def __init__(self, entry, args, keep, stream, device_index, out, lse):
        self._entry = entry
        self._fn = getattr(lib, entry)
        self._args = args
        self._ref = ctypes.byref(args)
        self._keep = keep
        self._stream = stream
        self._dev = device_index
        self.out, self.lse = out, lse

    def __call__(self):
        handle = self._stream.cuda_stream if self._stream is not None else _current_stream_handle(self._dev)
        st = self._fn(self._ref, ctypes.c_void_p(handle))
        if st != ATLAS_OK:
            raise AtlasError(st, self._entry)
        return self.out, self.lse


def prepare_attend(kind: str, q, k_pages, v_pages, page_table, context_lens, scale, *, out, lse=None,
                   workspace=None, stream=None, head_map=None, window=None, sink_tokens=None, softcap=None,
                   split_tokens=0) -> PreparedAttend:
    """A repeatable atlas_attend_decode (kind "decode") or atlas_attend_prefill
    (kind "prefill") call over fixed tensors: the checks and the argument
    structure are done here once (and the workspace allocated, if none is
    given), so each call costs only the C-ABI call.  For loops that reuse
    the same buffers with new contents.  `out` is required."""
    fns = {"decode": ("atlas_attend_decode", atlas_decode_workspace_bytes),
           "prefill": ("atlas_attend_prefill", atlas_prefill_workspace_bytes)}
    if kind not in fns:
        raise ValueError(f"kind must be 'decode' or 'prefill', got {kind!r}")
    entry, ws_fn = fns[kind]
    if out is None:
        raise ValueError("a prepared call writes to a fixed out tensor")
    args, keep = make_attn_args(q, k_pages, v_pages, page_table, context_lens, scale, head_map=head_map,
                                window=window, sink_tokens=sink_tokens, softcap=softcap, out=out, lse=lse,
                                split_tokens=split_tokens)
    dev = q.device
    if workspace is None:
        with (torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()):
            workspace = torch.empty(max(ws_fn(args), 1), dtype=torch.uint8, device=dev)
    else:
        _check(workspace, "workspace", None, dev)
    args.workspace = _ptr(workspace)
    args.workspace_bytes = workspace.numel() * workspace.element_size()
    keep += [q, k_pages, v_pages, page_table, context_lens, out, lse, workspace, window, sink_tokens, softcap]
    return PreparedAttend(entry, args, keep, stream, dev.index, out, lse)


def atlas_regenerate_pages(k_pages, v_pages, jobs, seed: int, layer: int = 0, stream=None):
    """Regenerate whole pages into the arenas.  jobs: int32 [n][3] device tensor of
    (seq, logical_page, phys_page)."""
    if k_pages.dtype not in _DTYPES:
        raise ValueError("arena dtype must be float32 or bfloat16")
    _check(k_pages, "k_pages", None, None, 4)
    _check(v_pages, "v_pages", k_pages.dtype, k_pages.device, 4)
    if v_pages.shape != k_pages.shape:
        raise ValueError("k_pages and v_pages must have the same shape")
    n_jobs = 0
    if jobs is not None and jobs.numel() > 0:
        _check(jobs, "jobs", torch.int32, k_pages.device, 2)
        if jobs.shape[1] != 3:
            raise ValueError("jobs must be [n][3] int32")
        n_jobs = jobs.shape[0]
    num_phys, hkv, P, d = k_pages.shape
    a = RegenArgs()
    a.seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    a.layer = int(layer)
    a.dtype = _DTYPES[k_pages.dtype]
    a.num_kv_heads, a.head_dim, a.page_size, a.num_phys_pages = hkv, d, P, num_phys
    a.num_jobs = n_jobs
    a.jobs = _ptr(jobs) if n_jobs else None
    a.k_pages, a.v_pages = _ptr(k_pages), _ptr(v_pages)
    st = lib.atlas_regenerate_pages(ctypes.byref(a), _stream(stream, k_pages.device))
    if st != ATLAS_OK:
        raise AtlasError(st, "atlas_regenerate_pages")


def atlas_append_kv(k_pages, v_pages, k_new, v_new, page_table, start_pos, stream=None):
    """Write new tokens' K/V rows (k_new, v_new [B][n_new][Hkv][D]) into their pages:
    token t of sequence b goes to position start_pos[b] + t (page_table[b][pos // P],
    row pos % P) in both arenas."""
    if k_pages.dtype not in _DTYPES:
        raise ValueError("arena dtype must be float32 or bfloat16")
    dev = k_pages.device
    _check(k_pages, "k_pages", None, dev, 4)
    _check(v_pages, "v_pages", k_pages.dtype, dev, 4)
    _check(k_new, "k_new", k_pages.dtype, dev, 4)
    _check(v_new, "v_new", k_pages.dtype, dev, 4)
    _check(page_table, "page_table", torch.int32, dev, 2)
    _check(start_pos, "start_pos", torch.int32, dev, 1)
    num_phys, hkv, P, d = k_pages.shape
    B, n_new, hk2, d2 = k_new.shape
    if v_pages.shape != k_pages.shape or v_new.shape != k_new.shape or hk2 != hkv or d2 != d:
        raise ValueError("k_new/v_new must be [B][n_new][Hkv][D] matching the arenas")
    if page_table.shape[0] != B or start_pos.shape[0] != B:
        raise ValueError("page_table and start_pos need one row per sequence")
    a = AppendArgs()
    a.dtype = _DTYPES[k_pages.dtype]
    a.batch, a.n_new, a.num_kv_heads, a.head_dim = B, n_new, hkv, d
    a.page_size, a.num_phys_pages, a.max_pages_per_seq = P, num_phys, page_table.shape[1]
    a.k_new, a.v_new = _ptr(k_new), _ptr(v_new)
    a.page_table, a.start_pos = _ptr(page_table), _ptr(start_pos)
    a.k_pages, a.v_pages = _ptr(k_pages), _ptr(v_pages)
    st = lib.atlas_append_kv(ctypes.byref(a), _stream(stream, k_pages.device))
    if st != ATLAS_OK:
        raise AtlasError(st, "atlas_append_kv")


class PagePool:
    """Host-side page pool (reference-counted physical page ids) of the C ABI."""

    def __init__(self, num_pages: int):
        h = ctypes.c_void_p()
        st = lib.atlas_pool_create(int(num_pages), ctypes.byref(h))
        if st != ATLAS_OK:
            raise AtlasError(st, "atlas_pool_create")
        self._h = h

    def close(self):
        if self._h:
            lib.atlas_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    @staticmethod
    def _ids(ids):
        ids = [int(i) for i in ids]
        return len(ids), (ctypes.c_int32 * max(len(ids), 1))(*ids)

    def alloc(self, n: int) -> list:
        buf = (ctypes.c_int32 * max(int(n), 1))()
        st = lib.atlas_pool_alloc(self._h, int(n), buf)
        if st != ATLAS_OK:
            raise AtlasError(st, "atlas_pool_alloc")
        return list(buf[:int(n)])

    def retain(self, ids):
        n, buf = self._ids(ids)
        st = lib.atlas_pool_retain(self._h, n, buf)
        if st != ATLAS_OK:
            raise AtlasError(st, "atlas_pool_retain")

    def release(self, ids):
        n, buf = self._ids(ids)
        st = lib.atlas_pool_release(self._h, n, buf)
        if st != ATLAS_OK:
            raise AtlasError(st, "atlas_pool_release")

    def free_pages(self) -> int:
        return int(lib.atlas_pool_free_pages(self._h))

    def refcount(self, page: int) -> int:
        return int(lib.atlas_pool_refcount(self._h, int(page)))


class HotCache:
    """Byte-bounded hot-page cache of the C ABI (atlas_cache_*): plans which
    pages of a call are resident (a hot-pool slot) and which are regenerated
    in the kernel (ATLAS_PAGE_REGENERATE)."""

    _h = None
    last_cold = 0   # pages the last plan left to in-kernel regeneration (0: plain decode gives the same bits)

    def __init__(self, hot_cache_bytes: int, page_bytes: int, page_size: int, recent_tokens: int = 0,
                 admit_regenerated: bool = True):
        cfg = CacheConfig(int(hot_cache_bytes), int(page_bytes), int(page_size), int(recent_tokens),
                          1 if admit_regenerated else 0, 0)
        h = ctypes.c_void_p()
        st = lib.atlas_cache_create(ctypes.byref(cfg), ctypes.byref(h))
        if st != ATLAS_OK:
            raise AtlasError(st, "atlas_cache_create")
        self._h = h

    def close(self):
        if self._h:
            lib.atlas_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def plan(self, layer: int, seq_ids, context_lens, max_pages_per_seq: int):
        """Returns (page_table int32 [B][max_pages_per_seq], jobs int32 [n][3]) as numpy arrays.
        seq_ids (distinct, in [0, 65536)) are also the sequences' generator keys: pass them as
        seq_keys to atlas_attend_decode_regen and the jobs to atlas_regenerate_pages."""
        import numpy as np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
        B = ids.shape[0]
        pt = np.empty((B, int(max_pages_per_seq)), dtype=np.int32)
        max_jobs = B * int(max_pages_per_seq)  # >= the pages of the call
        jobs = np.empty((max_jobs, 3), dtype=np.int32)
        n = ctypes.c_int32()
        n_cold = ctypes.c_int32()
        i32p, i64p = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
        st = lib.atlas_cache_plan(self._h, int(layer), B, ids.ctypes.data_as(i64p), ctx.ctypes.data_as(i32p),
                                  int(max_pages_per_seq), pt.ctypes.data_as(i32p), jobs.ctypes.data_as(i32p),
                                  max_jobs, ctypes.byref(n), ctypes.byref(n_cold))
        if st != ATLAS_OK:
            raise AtlasError(st, "atlas_cache_plan")
        self.last_cold = int(n_cold.value)
        return pt, jobs[:n.value].copy()

    def drop_sequence(self, seq_id: int):
        st = lib.atlas_cache_drop_sequence(self._h, int(seq_id))
        if st != ATLAS_OK:
            raise AtlasError(st, "atlas_cache_drop_sequence")

    def stats(self) -> dict:
        out = CacheStats()
        st = lib.atlas_cache_get_stats(self._h, ctypes.byref(out))
        if st != ATLAS_OK:
            raise AtlasError(st, "atlas_cache_get_stats")
        return {n: int(getattr(out, n)) for n, _ in CacheStats._fields_}

"""Exact causal grouped-query attention over a paged K/V cache on MI355X.

The computation lives in libatlas.so (hand-written HIP for gfx950 behind the
C ABI of include/atlas.h); this package is its Python binding.
"""
from .atlas import (  # noqa: F401
    ATLAS_DTYPE_BF16, ATLAS_DTYPE_F32, ATLAS_ERR_DEVICE, ATLAS_ERR_NONFINITE, ATLAS_ERR_NULL,
    ATLAS_ERR_POOL, ATLAS_ERR_RANGE, ATLAS_ERR_SHAPE, ATLAS_ERR_UNSUPPORTED, ATLAS_ERR_WORKSPACE,
    ATLAS_OK, ATLAS_PAGE_REGENERATE, AppendArgs, AtlasError, AttnArgs, AttnMods, CacheConfig, CacheStats, HotCache,
    PagePool, PreparedAttend, RegenArgs,
    atlas_abi_version, atlas_append_kv, atlas_attend_mods,
    atlas_attend_decode, atlas_attend_decode_noalloc, atlas_attend_decode_regen, atlas_attend_prefill,
    atlas_decode_workspace_bytes,
    atlas_last_error,
    atlas_prefill_workspace_bytes, atlas_regenerate_pages, atlas_status_str, make_attn_args,
    prepare_attend,
)

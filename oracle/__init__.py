"""fp64 CPU oracle for exact causal GQA attention over a K/V history.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  The product library never
imports this package, and this package imports nothing from the product.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over rows); this
module compiles it with gcc when needed and marshals numpy arrays.  Every
function cites the passage of the reference pages it follows in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "liboracle.so")
_lock = threading.Lock()
_lib = None

TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2


def build(force: bool = False) -> str:
    """Compile oracle.c into _build/liboracle.so (gcc, -O2, OpenMP, no fast-math)."""
    os.makedirs(_BUILD_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-std=c11", "-D_GNU_SOURCE", "-O2", "-ffp-contract=off", "-fopenmp",
               "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        lib = ctypes.CDLL(build())
        u32p = ctypes.POINTER(ctypes.c_uint32)
        lib.oracle_philox4x32_10_batch.argtypes = [ctypes.c_int64, u32p, u32p, u32p]
        lib.oracle_philox4x32_10_batch.restype = None
        lib.oracle_regen_value.argtypes = [ctypes.c_uint64] + [ctypes.c_uint32] * 6
        lib.oracle_regen_value.restype = ctypes.c_double
        lib.oracle_regen_rows.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                          ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int64,
                                          ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.oracle_regen_rows.restype = None
        lib.oracle_attend_mods.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double,
                                           ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                           ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                           ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_attend_mods.restype = ctypes.c_int
        lib.oracle_attend.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                      ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_attend.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
        return lib


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def philox4x32_10(ctrs, key) -> np.ndarray:
    """Philox4x32-10 bijection (Salmon et al., SC'11) on counters [n][4] under key (k0, k1)."""
    lib = _load()
    c = np.ascontiguousarray(np.asarray(ctrs, dtype=np.uint32).reshape(-1, 4))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32).reshape(2))
    out = np.empty_like(c)
    u32p = ctypes.POINTER(ctypes.c_uint32)
    lib.oracle_philox4x32_10_batch(c.shape[0], c.ctypes.data_as(u32p), k.ctypes.data_as(u32p),
                                   out.ctypes.data_as(u32p))
    return out


def regen_value(seed: int, layer: int, seq: int, tensor: int, head: int, token: int, dim: int) -> float:
    """One regenerated value in fp64, before rounding to the storage type."""
    return float(_load().oracle_regen_value(seed, layer, seq, tensor, head, token, dim))


def regen_rows(seed: int, layer: int, seq: int, tensor: int, head: int, t0: int, n_tokens: int,
               dims: int, kind: str = "f32") -> np.ndarray:
    """Rows [t0, t0+n_tokens) x dims of one regenerated stream.

    kind: "f64" (unrounded), "f32" (fp32 RNE), "bf16" (uint16 bit patterns,
    fp32 value rounded RNE to bf16)."""
    lib = _load()
    code, dt = {"f64": (0, np.float64), "f32": (1, np.float32), "bf16": (2, np.uint16)}[kind]
    out = np.empty((n_tokens, dims), dtype=dt)
    lib.oracle_regen_rows(seed, layer, seq, tensor, head, t0, n_tokens, dims, code,
                          out.ctypes.data)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to fp32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def attend(q, k, v, pos, head_map, scale: float, window: int = 0, n_sinks: int = 0,
           softcap: float = 0.0, causal: bool = True, alibi=None, mask=None, allow_empty: bool = False):
    """Full-KV attention for one sequence in fp64 (two-pass softmax).

    q [nq][hq][D], k/v [hkv][n_kv][D] (fp32 arrays; bf16 data widened
    exactly), pos [nq] absolute query positions, head_map [hq].  causal=False
    lets every row see all n_kv keys; alibi [hq] adds -slope * |pos - j| to
    each logit (after the softcap); mask [nq][n_kv] (booleans) additionally
    hides keys; allow_empty makes rows with no visible key NaN (lse -inf)
    instead of an error.  Returns (out [nq][hq][D] fp64, lse [nq][hq] fp64)."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    pos = np.ascontiguousarray(pos, dtype=np.int32).reshape(-1)
    hm = np.ascontiguousarray(head_map, dtype=np.int32).reshape(-1)
    nq, hq, dims = q.shape
    hkv, n_kv, dk = k.shape
    if v.shape != k.shape or dk != dims or pos.shape[0] != nq or hm.shape[0] != hq:
        raise ValueError("oracle.attend: inconsistent shapes")
    al = None if alibi is None else np.ascontiguousarray(alibi, dtype=np.float64).reshape(-1)
    if al is not None and al.shape[0] != hq:
        raise ValueError("oracle.attend: alibi needs one slope per q-head")
    mk = None if mask is None else np.ascontiguousarray(mask, dtype=bool).astype(np.uint8)
    if mk is not None and mk.shape != (nq, n_kv):
        raise ValueError("oracle.attend: mask must be [nq][n_kv]")
    out = np.empty((nq, hq, dims), dtype=np.float64)
    lse = np.empty((nq, hq), dtype=np.float64)
    rc = lib.oracle_attend_mods(nq, pos.ctypes.data, n_kv, hq, hkv, dims, q.ctypes.data, k.ctypes.data,
                                v.ctypes.data, hm.ctypes.data, float(scale), int(window), int(n_sinks),
                                float(softcap), 1 if causal else 0,
                                None if al is None else al.ctypes.data,
                                None if mk is None else mk.ctypes.data, 1 if allow_empty else 0,
                                out.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise ValueError("oracle.attend: empty visible set or position out of range")
    return out, lse


def default_head_map(hq: int, hkv: int) -> np.ndarray:
    """Contiguous GQA grouping: q-head h reads K/V head h // (hq // hkv)."""
    return np.arange(hq, dtype=np.int32) // (hq // hkv)


def gather_pages(arena, page_table_row, n_tokens: int, page_size: int) -> np.ndarray:
    """Unpaged history [H][n_tokens][D] of one sequence from a physical arena
    [num_phys][H][page_size][D] and its logical->physical page list (plain
    indexing; the CFR-Atlas README's "Core contract" compares the folded result
    against attention over exactly these rows)."""
    arena = np.asarray(arena)
    n_pages = -(-n_tokens // page_size)
    ids = np.asarray(page_table_row[:n_pages], dtype=np.int64)
    pages = arena[ids]                                  # [n_pages][H][P][D]
    h = pages.shape[1]
    rows = pages.transpose(1, 0, 2, 3).reshape(h, n_pages * page_size, pages.shape[3])
    return np.ascontiguousarray(rows[:, :n_tokens, :])

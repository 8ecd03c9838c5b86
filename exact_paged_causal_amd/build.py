"""Build libatlas.so in-tree with hipcc for gfx950.

Every HIP source under csrc/ is compiled to an object file (in parallel) and
linked into exact_paged_causal_amd/libatlas.so.  Run as a module or call
build().
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import hashlib
import json
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libatlas.so")
INFO = os.path.join(HERE, "build_info.json")   # written beside the library (not committed)
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # Packed-fp32 VALU forms stay disabled for every kernel.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, hipcc: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc, *FLAGS, *extra, "-x", "hip", "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return obj


def sources_sha256() -> str:
    """Hash of the library's sources (csrc and the public header)."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(CSRC, "*")) + [os.path.join(INCLUDE, "atlas.h")])
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _git(*args):
    try:
        r = subprocess.run(["git", "-C", os.path.dirname(HERE), *args], capture_output=True, text=True, timeout=10)
        return r.stdout.strip() if r.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        return None


def build(verbose: bool = False, extra=()) -> str:
    """Compile every csrc/*.hip and csrc/*.cpp and link libatlas.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    workers = min(len(sources), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc, list(extra)), sources))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    status = _git("status", "--porcelain", "--", "exact_paged_causal_amd/csrc", "include")
    info = {"git_commit": _git("rev-parse", "HEAD"),
            "sources_modified_since_commit": None if status is None else bool(status),
            "sources_sha256": sources_sha256(), "hipcc_flags": FLAGS + list(extra)}
    with open(INFO, "w") as f:
        json.dump(info, f, indent=1)
    if verbose:
        print(f"built {LIB} from {len(sources)} sources")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])

"""Builds libqsa.so (the HIP library) for gfx950 with hipcc, in-tree.

Usage: python -m block_sparse_attention_32_amd.build [--verbose] [--incremental] [--debug]

--debug builds libqsa_debug.so: the same sources with -DQSA_DEBUG (device
data checks, see qsa_debug_take in include/qsa.h).

--incremental recompiles only the sources whose object is older than the
source or than any header of csrc/ and include/ (a full build otherwise).
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqsa.so")
# the same sources with the device-data checks on (-DQSA_DEBUG)
DEBUG_LIB = os.path.join(PKG, "libqsa_debug.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    if os.path.exists(path):
        return path
    found = shutil.which("hipcc")
    if not found:
        raise RuntimeError("hipcc not found (ROCm is required to build libqsa)")
    return found


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _headers_mtime() -> float:
    hs = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hpp", ".h"))]
    hs += [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h")]
    return max(os.path.getmtime(h) for h in hs)


def _compile(src: str, verbose: bool, newest_dep: float = None, debug: bool = False) -> str:
    obj = os.path.join(BUILD, "debug" if debug else "", os.path.basename(src) + ".o")
    if newest_dep is not None and os.path.exists(obj) and \
            os.path.getmtime(obj) > max(newest_dep, os.path.getmtime(src)):
        return obj
    cmd = [hipcc(), *HIPCC_FLAGS, *(["-DQSA_DEBUG"] if debug else []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(verbose: bool = False, incremental: bool = False, debug: bool = False) -> str:
    """Compile every csrc/*.hip for gfx950 and link libqsa.so (debug:
    libqsa_debug.so with -DQSA_DEBUG); returns its path."""
    out_dir = os.path.join(BUILD, "debug") if debug else BUILD
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    dep = _headers_mtime() if incremental else None
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, dep, debug), srcs))
    stale = set(os.listdir(out_dir)) - {os.path.basename(o) for o in objs}
    for f in stale:  # objects of removed sources
        if f.endswith(".hip.o"):
            os.remove(os.path.join(out_dir, f))
    lib = DEBUG_LIB if debug else LIB
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv, incremental="--incremental" in sys.argv,
                debug="--debug" in sys.argv))

"""Build libssm_hip.so (the C-ABI HIP library) in-tree for gfx950.

    python -m selective_state_space_59_amd.build

Each source is compiled by hipcc to an object under _build/ (in parallel),
then linked into selective_state_space_59_amd/libssm_hip.so.  Every call
compiles from scratch, so the result always matches the sources.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libssm_hip.so")
ARCH = "gfx950"

SOURCES = ["ssm_api.cpp", "scan_fwd.hip", "scan_bwd.hip", "conv1d.hip", "state_update.hip", "block.hip",
           "ssd.hip", "scan_noalloc.hip"]
# hipBLASLt runs the plain GEMMs of the Mamba block.
LIBS = ["-L/opt/rocm/lib", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib"]

# Packed-fp32 VALU forms are switched off for all device code; the compiler
# still emits ordinary fp32 arithmetic.
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-x", "hip",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-I", os.path.join(PKG, "..", "include")]


def _code_only(text: bytes) -> bytes:
    """Source text without comments and blank space (comments do not change a build)."""
    import re
    t = text.decode("utf-8")
    t = re.sub(r"/\*.*?\*/", " ", t, flags=re.S)
    t = re.sub(r"//[^\n]*", " ", t)
    return " ".join(t.split()).encode()


def source_hash(sources=None) -> str:
    """sha256 over the code (comments excluded) of the library sources `sources` (file
    names under csrc/) and the compile flags, or of every library source and the public
    header when None: it identifies a kernel build for measurements taken on it."""
    import hashlib
    h = hashlib.sha256()
    names = sorted(os.listdir(CSRC)) if sources is None else sorted(sources)
    if sources is not None:  # the flags, less the include path (it differs between checkouts)
        flags = [f for i, f in enumerate(COMMON) if f != "-I" and (i == 0 or COMMON[i - 1] != "-I")]
        h.update(" ".join(flags).encode() + b"\0")
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(n.encode() + b"\0" + _code_only(f.read()))
    if sources is None:
        with open(os.path.join(PKG, "..", "include", "ssm.h"), "rb") as f:
            h.update(_code_only(f.read()))
    return h.hexdigest()[:16]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs + LIBS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

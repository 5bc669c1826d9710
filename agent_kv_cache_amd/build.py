"""Build libakv.so in-tree with hipcc for gfx950.

    python -m agent_kv_cache_amd.build

Each .hip file is compiled to an object in parallel, then linked into
agent_kv_cache_amd/libakv.so.  Packed fp32 instructions are disabled for all
device code (-target-feature -packed-fp32-ops).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libakv.so")
SOURCES = ["akv_host.hip", "akv_compact.hip", "akv_move.hip", "akv_attn.hip", "akv_segment.hip"]
ARCH = os.environ.get("AKV_OFFLOAD_ARCH", "gfx950")


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-result"]


def build(verbose: bool = False, defines=(), out: str = LIB, tag: str = "") -> str:
    """Compile and link; `defines` are extra -D macros (launch-shape knobs)."""
    bdir = os.path.join(BUILD, tag) if tag else BUILD
    os.makedirs(bdir, exist_ok=True)
    hipcc = _hipcc()
    dflags = [f"-D{x}" for x in defines]

    def compile_one(src):
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        cmd = [hipcc, *common_flags(), *dflags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build libsparse3d.so in-tree for gfx950 with hipcc.

Run as ``python -m dynamic_block_sparse_tile_amd.build``.  Every call compiles
every source again (objects go to ``_build/`` at the repository root), then links
``dynamic_block_sparse_tile_amd/libsparse3d.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsparse3d.so")

SOURCES = ["validate.cpp", "api.hip", "pool_score.hip", "topk.hip", "attn.hip", "attn_bf16.hip", "attn_bwd.hip",
           "subsample.hip"]

ARCH = os.environ.get("SPARSE3D_ARCH", "gfx950")
# Packed fp32 VALU ops are disabled in device code (the compiler would otherwise form
# v_pk_* from ordinary float code); the host pass warns that it does not know the feature.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError("hipcc not found (ROCm is required to build the library)")
    return cand


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [hipcc(), f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, "-c", path, "-o", obj]
    else:
        cmd = [hipcc(), *COMMON, "-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if ln.strip() and noise not in ln]
    if msgs:
        print(f"[build] {src}:\n" + "\n".join(msgs), file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"[build] {LIB}")
    return LIB


if __name__ == "__main__":
    build()

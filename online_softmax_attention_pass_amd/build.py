"""Compile the HIP sources into the in-tree shared library ``librf.so`` (gfx950 only).

Run as ``python -m online_softmax_attention_pass_amd.build``. Objects go to
``_build/`` at the repository root; the library lands next to this file so
that the binding loads it from the package directory.
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
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librf.so")
ARCH = "gfx950"

SOURCES = [
    "rf_api.cpp",
    "softmax_rows.hip",
    "layernorm_rows.hip",
    "lse_merge.hip",
    "decode_splitkv.hip",
    "decode_noalloc.hip",
    "attention_f32.hip",
    "attention_bf16.hip",
    "moe_route.hip",
    "attention_rowwise.hip",
]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-variable",
    f"-I{INCLUDE}", f"-I{CSRC}",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _compile(src: str, verbose: bool, defines=(), objdir: str = OBJDIR) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-x", "hip", f"--offload-arch={ARCH}", *COMMON, *[f"-D{d}" for d in defines], "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(verbose: bool = False, defines=(), out: str = LIB, objdir: str = OBJDIR) -> str:
    """Compile and link. ``defines`` are NAME=VALUE compile-time knobs (tuning
    variants); ``out`` / ``objdir`` place a variant library elsewhere."""
    os.makedirs(objdir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, defines, objdir), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking librf.so failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

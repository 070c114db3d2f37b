"""Builds libiq.so (the HIP/gfx950 library behind include/iq.h) in-tree.

    python -m compressed_space_attention_isoquant_amd.build

Each source compiles to an object under ``_build/`` in parallel; the objects
link into ``compressed_space_attention_isoquant_amd/lib/libiq.so``.
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
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libiq.so")

SOURCES = ["api.cpp", "quantize.hip", "decode.hip", "decode_128.hip", "decode_256.hip", "decode_512.hip",
           "noalloc.hip"]

# Matrix-core accumulators kept in the unified VGPR file (no AGPR copies around
# the value accumulators).  Not for head_dim 512, whose register pressure makes
# this compiler's AGPR-rewrite pass fail.
EXTRA = {
    "decode_128.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "decode_256.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}

# gfx950 only.  Packed-fp32 instruction selection is switched off for device
# code (the host pass warns that it does not know the feature; harmless).
COMMON = [
    "-O3", "-fPIC", "-std=c++17", "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)

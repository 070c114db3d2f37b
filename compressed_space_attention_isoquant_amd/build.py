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

SOURCES = ["api.cpp", "quantize.hip", "decode.hip", "decode_128.hip", "decode_256.hip", "decode_512.hip", "probe.hip",
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


# The host-side argument checks of api.cpp built with AddressSanitizer and
# UndefinedBehaviorSanitizer (host code only, by the LLVM that ships with
# ROCm, as plain C++), linked with the device objects of build().  Loaded into
# a Python process, it needs the sanitizer runtime preloaded (LD_PRELOAD).
HOSTSAN_LIB = os.path.join(BUILD, "libiq_hostsan.so")


def _rocm_clang() -> str:
    for cand in ("/opt/rocm/llvm/bin/clang++", "/opt/rocm/lib/llvm/bin/clang++"):
        if os.path.exists(cand):
            return cand
    raise RuntimeError("ROCm clang++ not found")


def hostsan_runtime() -> str:
    """Path of the ASan runtime the sanitized library links against."""
    r = subprocess.run([_rocm_clang(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True, check=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("ASan runtime not found")
    return path


def build_host_sanitized() -> str:
    objs = [os.path.join(BUILD, s + ".o") for s in SOURCES if s != "api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        build(verbose=False)
    clang = _rocm_clang()
    api_obj = os.path.join(BUILD, "api_hostsan.o")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libsan"]
    cmd = [clang, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{INCLUDE}", f"-I{CSRC}",
           "-fPIC", "-g", "-O1", "-fno-omit-frame-pointer", *san, "-c", os.path.join(CSRC, "api.cpp"), "-o", api_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized compile of api.cpp failed:\n{r.stderr}")
    cmd = [clang, "-shared", "-fPIC", *san, api_obj, *objs, "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib", "-o", HOSTSAN_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    return HOSTSAN_LIB


if __name__ == "__main__":
    build()
    sys.exit(0)

"""Build the HIP library ``libmla.so`` for gfx950 in-tree with hipcc.

Usage: ``python -m mla_latent_kv_decode_amd.build`` (or ``build()`` from Python).
Every source is compiled on every call (this is the "does it build" check);
objects go to ``_build/`` and the shared library next to this file.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmla.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["mla.cpp", "k_generic.hip", "k_gemm.hip", "k_gemm_big.hip", "k_decode_wide.hip", "k_decode_ring.hip", "k_decode_ring8.hip", "k_combine.hip", "k_skinny.hip", "k_prefill.hip", "k_gather.hip", "scratch.hip"]

ARCH = "gfx950"
# -packed-fp32-ops: hipcc must not emit packed fp32 ALU ops by itself (its host
# pass warns that it does not know the feature; harmless).
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", f"-I{os.path.join(ROOT, 'include')}"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the MLA library)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = OUT + ".tmp"
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "lib")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp,
           f"-Wl,-rpath,{rocm_lib}"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


# Host-side sanitizers for the C-ABI's host logic (argument checks, work
# planning, layouts): mla.cpp is rebuilt with AddressSanitizer and
# UndefinedBehaviorSanitizer on its host pass only (GPU code is never built
# with them) and linked with the kernel objects of the normal build.  The
# result loads only into a process that has the ASan runtime first in its
# library list (LD_PRELOAD=asan_runtime()).
SAN_DIR = os.path.join(BUILD_DIR, "san")
SAN_OUT = os.path.join(SAN_DIR, "libmla_san.so")
SAN_FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument", f"-I{os.path.join(ROOT, 'include')}",
             "-Xarch_host", "-fsanitize=address,undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """Path of the compiler's shared ASan runtime (it carries the UBSan
    handlers too)."""
    llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "llvm")
    for cand in sorted(glob.glob(os.path.join(llvm, "lib", "clang", "*", "lib", "linux",
                                              "libclang_rt.asan-x86_64.so"))):
        return cand
    raise RuntimeError("the ASan runtime of the ROCm compiler was not found")


def build_sanitized(verbose: bool = False) -> str:
    os.makedirs(SAN_DIR, exist_ok=True)
    objs = []
    for src in SOURCES:
        if src == "mla.cpp":
            continue
        obj = os.path.join(BUILD_DIR, src + ".o")
        objs.append(obj if os.path.exists(obj) else _compile(src, verbose))
    host = os.path.join(SAN_DIR, "mla.cpp.o")
    cmd = [hipcc(), *SAN_FLAGS, "-c", os.path.join(CSRC, "mla.cpp"), "-o", host]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on mla.cpp (sanitized):\n{r.stdout}\n{r.stderr}")
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "lib")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", host, *objs, "-o", SAN_OUT,
           f"-Wl,-rpath,{rocm_lib}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed (sanitized):\n{r.stdout}\n{r.stderr}")
    return SAN_OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

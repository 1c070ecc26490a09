"""Build libuw.so (host codec + C ABI + gfx950 kernels) in-tree with hipcc.

Usage: ``python decode_gemm_bf16_amd/build.py`` (run by path: importing the
package would load the library before it exists).
Every source is compiled for gfx950 only; the library links hipBLASLt for the
plain GEMM of pipeline 1.  Objects go to ``_build/`` next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libuw.so")
BUILD = os.path.join(HERE, "_build")

SOURCES = ["codec.cpp", "runtime.cpp", "variants.cpp", "fused_small.hip", "fused_mid.hip", "fused_large.hip", "fused_ring.hip", "fused_wide.hip", "fused_rowk.hip", "transcode.hip",
           "huff_decode.hip", "misc.hip", "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-mcode-object-version=5", "-I", os.path.join(ROOT, "include"),
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-function",
          "-Wno-unused-variable", "-Wno-unused-but-set-variable"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _torch_lib() -> str:
    """Directory of the HIP runtime that PyTorch loads.  The library links that
    same runtime (libamdhip64.so, libhipblaslt.so by soname) so that torch's
    device memory and streams are valid in it: two HIP runtimes in one process
    do not share devices."""
    import torch
    return os.path.join(os.path.dirname(torch.__file__), "lib")


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libuw.so.  Returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    workers = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    tl = _torch_lib()
    cmd = ["g++", "-shared", "-fPIC", *objs, "-o", tmp, f"-L{tl}", "-l:libamdhip64.so", "-l:libhipblaslt.so",
           f"-Wl,-rpath,{tl}", "-Wl,--no-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)

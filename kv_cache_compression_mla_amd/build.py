"""Build libmla.so in-tree with hipcc for gfx950 (host code and kernels)."""
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
LIB = os.path.join(PKG, "libmla.so")
# measurement build: the same sources with per-workgroup clock stamps in the
# attention kernel (clock_stamps.py beside bench.py reads them)
LIB_STAMPS = os.path.join(PKG, "libmla_stamps.so")
SOURCES = ["attn_mfma.hip", "attn_generic.hip", "attn_prefill.hip", "gemm.hip", "mla_api.cpp"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-I" + INCLUDE, "-I" + CSRC,
    # packed fp32 VALU forms are kept out of all generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False, stamps: bool = False) -> str:
    """Build libmla.so (or, with stamps, the measurement build libmla_stamps.so)."""
    objdir = os.path.join(PKG, "_build_stamps" if stamps else "_build")
    os.makedirs(objdir, exist_ok=True)
    extra = ["-DMLA_CLOCK_STAMPS"] if stamps else []
    target = LIB_STAMPS if stamps else LIB

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"]
        cmd = [HIPCC, *FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = target + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, target)
    return target


if __name__ == "__main__":
    print(build(verbose=True))
    print(build(verbose=True, stamps=True))

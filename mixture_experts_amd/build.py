"""Compile the gfx950 HIP library libmoe_mi355x.so in-tree with hipcc.

Also builds libmoe_mi355x_flatcopy.so, the same library with the GEMM kernels'
64-bit (FLAT) LDS-copy form forced on (MOE_FORCE_FLAT_COPIES=1), which the GPU
tests run to exercise that form; the product loads libmoe_mi355x.so.

Usage: python -m mixture_experts_amd.build   (or build() from Python)
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe_mi355x.so")
FLAT_LIB = os.path.join(PKG, "libmoe_mi355x_flatcopy.so")
SOURCES = ["moe_api.hip", "route.hip", "permute.hip", "ffn_rs.hip", "ffn_misc.hip", "ffn_lds.hip", "norm.hip",
           "convert.hip", "noalloc.hip"]
FLAT_SOURCES = ["ffn_rs.hip", "ffn_lds.hip"]          # the files MOE_FORCE_FLAT_COPIES changes

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # no packed-fp32 VALU instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc", "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, flat: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ("_flat.o" if flat else ".o"))
    cmd = [HIPCC, *FLAGS, *(["-DMOE_FORCE_FLAT_COPIES=1"] if flat else []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip():
        sys.stderr.write(r.stderr)
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(src, False) for src in SOURCES] + [(src, True) for src in FLAT_SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    main = objs[:len(SOURCES)]
    flat = {src: o for (src, _), o in zip(jobs[len(SOURCES):], objs[len(SOURCES):])}
    _link(main, LIB)
    _link([flat.get(src, o) for src, o in zip(SOURCES, main)], FLAT_LIB)
    if verbose:
        print(f"built {LIB} and {os.path.basename(FLAT_LIB)}")
    return LIB


if __name__ == "__main__":
    build()

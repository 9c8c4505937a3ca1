"""Builds libskv.so for gfx950 in-tree: hipcc compiles each source, g++ links the objects
against the HIP runtime that PyTorch ships, so that the library and torch share one runtime
(device pointers and streams from torch are valid in the library)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libskv.so")
# reference kernels for the benchmark's bandwidth ceilings (not part of the decode path)
REF_SOURCES = ["reference.hip"]
REF_LIB = os.path.join(PKG, "libskv_ref.so")
SOURCES = ["meta.hip", "score.hip", "select.hip", "attn.hip", "noalloc.hip", "abi.cpp"]
ARCH = os.environ.get("SKV_OFFLOAD_ARCH", "gfx950")


def _torch_lib_dir() -> str:
    import torch
    return os.path.join(os.path.dirname(torch.__file__), "lib")


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
           # packed fp32 (v_pk_*_f32) disabled in device code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, out: str):
    tlib = _torch_lib_dir()
    tmp = out + ".tmp"
    cmd = ["g++", "-shared", "-o", tmp] + objs + [f"-L{tlib}", "-l:libamdhip64.so", f"-Wl,-rpath,{tlib}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + REF_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in REF_SOURCES], REF_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)

"""Build libpagedkv.so (HIP for gfx950) in-tree with hipcc.

Usage: python pagedattention_decode_paged_amd/build.py [--jobs N] [--keep-asm DIR]
(run as a file: importing the package loads the library being rebuilt)
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpagedkv.so")

SOURCES = ["pagedkv_api.cpp", "block_allocator.cpp", "cache_kernels.hip", "decode_gqa.hip", "decode_gqa_ring.hip", "decode_int8.hip", "decode_mla.hip", "prefill_paged.hip", "probes.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 ops (v_pk_*_f32) stay off: the compiler must not form them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
]


def _compile(src: str, asm_dir: str | None) -> str:
    out_dir = asm_dir if (asm_dir and src.endswith(".hip")) else BUILD
    os.makedirs(out_dir, exist_ok=True)
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *lang, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if out_dir != BUILD:
        cmd.append("-save-temps=obj")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 4, asm_dir: str | None = None, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, asm_dir), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--keep-asm", default=None)
    a = ap.parse_args()
    build(a.jobs, a.keep_asm)

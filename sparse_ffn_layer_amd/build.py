"""Build the HIP library libsfl_moe.so in-tree for gfx950.

Every call compiles all sources (one hipcc process per file, in parallel) and
links them into sparse_ffn_layer_amd/libsfl_moe.so.  No GPU is needed: hipcc
cross-compiles the device code.

usage: python -m sparse_ffn_layer_amd.build [-j N] [--asm]
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
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsfl_moe.so")
SOURCES = ["api.cpp", "router.hip", "permute.hip", "gemm.hip", "combine.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the MoE library)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            # gfx950 packed-fp32 instructions are disabled for all device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


def _compile(src: str, asm: bool) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJ, src + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", path, "-o", obj] + common_flags()
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if asm and src.endswith(".hip"):
        s = os.path.join(OBJ, src + ".s")
        subprocess.run([hipcc(), "-x", "hip", "-S", "--cuda-device-only", path, "-o", s] + common_flags(),
                       check=True, capture_output=True)
    return out


def build(jobs: int = 0, asm: bool = False, verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        for src, out in zip(SOURCES, ex.map(lambda s: _compile(s, asm), SOURCES)):
            if verbose and out:
                print(f"[{src}]\n{out}", file=sys.stderr)
    objs = [os.path.join(OBJ, s + ".o") for s in SOURCES]
    tmp = LIB + ".tmp"
    r = subprocess.run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=0)
    ap.add_argument("--asm", action="store_true", help="also write device assembly to _build/")
    ap.add_argument("-v", action="store_true")
    a = ap.parse_args()
    print(build(a.j, a.asm, a.v))

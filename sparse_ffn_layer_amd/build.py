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
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsfl_moe.so")
SOURCES = ["api.cpp", "noalloc.hip", "router.hip", "capacity.hip", "permute.hip", "quant.hip", "gemm.hip",
           "combine.hip"]
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


def _check_no_scratch(src: str, remarks: str) -> None:
    """Fail if a GEMM kernel uses scratch (register spills).

    The GEMM kernels read their MFMA fragments with inline-asm LDS loads and
    wait for them explicitly; a spill would copy such a register before the
    data has arrived, so a spilling GEMM kernel is a build error, not a slow
    kernel."""
    name = None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and "grouped_gemm_bf16" in name and int(m.group(1)) > 0:
            raise RuntimeError(f"{src}: kernel {name} spills ({m.group(1)} scratch bytes/lane)")


def _compile(src: str, asm: bool) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJ, src + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", path, "-o", obj] + common_flags()
    if src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                        if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l and l.strip())
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    _check_no_scratch(src, r.stderr)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l and l.strip()
                    and not l.lstrip().startswith(("|", "^")) and not re.match(r"^\s*\d+ \|", l))
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

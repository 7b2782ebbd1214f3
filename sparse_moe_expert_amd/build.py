"""Build libmoe.so (gfx950) in-tree with hipcc.

    python -m sparse_moe_expert_amd.build        # or build() from Python

Every HIP source compiles to an object under _build/ (in parallel), then links
into sparse_moe_expert_amd/libmoe.so next to this file.  No torch extension
machinery: the library is plain C ABI and is loaded with ctypes.
"""
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")
ARCH = "gfx950"

SOURCES = ["moe_api.hip", "gemm.hip", "gemm_prefill.hip", "gemm_big.hip", "gemm_fp8.hip", "gemm_decode.hip", "route.hip", "dispatch.hip",
           "combine.hip", "norm.hip", "fused.hip", "pack.hip", "probe.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep hipcc from forming packed fp32 VALU ops (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the MoE library needs ROCm's hipcc to build")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link libmoe.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    headers = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    headers.append(os.path.join(INCLUDE, "moe.h"))

    def compile_one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmd = [cc, *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c",
               os.path.join(CSRC, src), "-o", obj]
        out = _run(cmd)
        if verbose and out.strip():
            print(out)
        return obj

    jobs = min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)

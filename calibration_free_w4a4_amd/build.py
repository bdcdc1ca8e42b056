"""Builds liborbq.so (the C-ABI library) in-tree for gfx950 with hipcc.

    python -m calibration_free_w4a4_amd.build      # or __graft_entry__.build()

Every HIP source gets -Xclang -target-feature -Xclang -packed-fp32-ops: the kernels are
written for unpacked fp32 VALU arithmetic.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liborbq.so")
ARCH = os.environ.get("ORBQ_OFFLOAD_ARCH", "gfx950")

SOURCES = ["lut_gemm_a4.hip", "lut_gemm_a6.hip", "lut_gemm_abf.hip", "lut_gemm_a2.hip", "lut_gemm_a3.hip",
           "rpbh_quantize_b128.hip", "rpbh_quantize_b64.hip", "rpbh_quantize_b256.hip", "rpbh_quantize_b512.hip",
           "rpbh_quantize_b1024.hip", "rpbh_quantize_b2048.hip", "rpbh_quantize_b4096.hip", "rpbh_quantize.hip", "a16_gemm.hip", "lut_gemm.hip", "flatness.hip", "noalloc.hip", "mfma_probe.hip",
           "api.cpp",
           "codebook.cpp"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc(), "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"-I{ROOT}/include", "-c", path, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = [f"--offload-arch={ARCH}", "-x", "hip", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    else:
        cmd[1:1] = ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

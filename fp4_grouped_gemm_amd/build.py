"""Build libfgg.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m fp4_grouped_gemm_amd.build        (or fp4_grouped_gemm_amd.build.build())

Every source is compiled with hipcc for gfx950 only; packed FP32 VALU
instructions are disabled (-packed-fp32-ops) and MFMA results are kept in
VGPRs (-amdgpu-mfma-vgpr-form).  Objects go to _build/ at the
repository root, the shared library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfgg.so")

SOURCES = ["api.cpp", "fp8_grouped.hip", "fp4.hip", "quant.hip", "w4a16.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the FP8 kernel promotes every partial with VALU
    # FMAs, which cannot read AGPRs directly.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    out = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return out


PROBES = ["mfma_peak", "lds_banks"]
PROBE = os.path.join(ROOT, "bench", "mfma_peak")


def build_probe(verbose: bool = False) -> str:
    """Build the microbenchmarks in bench/ (standalone HIP programs, not part
    of the library): mfma_peak (roofline legs) and lds_banks (LDS
    bank-conflict patterns)."""
    for name in PROBES:
        src = os.path.join(ROOT, "bench", name + ".hip")
        exe = os.path.join(ROOT, "bench", name)
        cmd = [HIPCC, *[f for f in FLAGS if f not in ("-fPIC",) and not f.startswith("-I")],
               src, "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        if verbose:
            print("built", exe)
    return PROBE


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

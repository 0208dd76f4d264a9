"""Build libpion_prefix.so (HIP kernels + C ABI) for gfx950 in-tree with hipcc.

Every HIP source is compiled with packed-fp32 instructions disabled (the compiler
would otherwise pair fp32 ops into v_pk_*_f32 forms) and linked into one shared
library next to this file, where the Python binding loads it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpion_prefix.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["attn_partial.hip", "attn_mlx4.hip", "attn_mlx4_mfma.hip", "attn_gqa_mfma.hip", "prefill_mfma.hip", "mlx4g32.hip", "sparse.hip", "vstore.hip", "stream_read.hip", "mfma_peak.hip", "noalloc.hip", "pion_prefix.cpp"]

COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          "-Wall", "-Wno-unused-function"]
DEVICE_ONLY = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               # kernels with scalar arguments receive them in SGPRs at launch (gfx950
               # kernel-argument preload) instead of loading them first; the compiler
               # also emits the loads for a loader that does not preload
               "-mllvm", "-amdgpu-kernarg-preload-count=16"]
# Inline assembly that writes M0 (the LDS-writing loads of mfma_common.h) saves and
# restores it in the same statement; a new use of M0 in inline assembly must do the same.


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON]
    if src.endswith(".hip"):
        # resource remarks: a kernel that spills registers to scratch is reported below
        cmd += DEVICE_ONLY + ["-x", "hip", "-Rpass-analysis=kernel-resource-usage"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    # vector registers spilled to scratch memory (scalar spills go to vector lanes)
    spills = [ln for ln in r.stderr.splitlines()
              if "VGPRs Spill:" in ln and "VGPRs Spill: 0 " not in ln]
    if spills:
        print(f"warning: {src}: a kernel spills vector registers to scratch (slow):\n  "
              + "\n  ".join(spills), file=sys.stderr)
    return obj


def build(jobs: int = 4) -> str:
    """Compile every source and link the library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())

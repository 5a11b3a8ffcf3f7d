"""Builds ``libsparse_moe.so`` (HIP kernels + C ABI) in-tree for gfx950.

Every source is compiled by hipcc for gfx950 only, with packed-fp32 VALU
instructions disabled, then linked into one shared library next to this file.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsparse_moe.so")
# measurement kernels (peak rates of the chip), a library of their own
PEAKS_SRC = os.path.join(PKG, "peaks", "peaks.hip")
PEAKS_LIB = os.path.join(PKG, "libmoe_peaks.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-x", "hip",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


# per-source extra flags: the GEMMs keep MFMA results in VGPRs (the fp32
# promotion reads them right away; the AGPR form would add one copy per value),
# and their atomics stay as written: one lane adds and its result is used only
# later (the wave-wide rewrite of the atomic optimizer would wait for the
# result, and with it for every load in flight, right after the atomic)
EXTRA = {"gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj, r.stderr


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    for _, err in results:
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    tmp = PEAKS_LIB + ".tmp"
    r = subprocess.run([HIPCC, *FLAGS, "-shared", PEAKS_SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PEAKS_SRC}:\n{r.stderr}")
    os.replace(tmp, PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

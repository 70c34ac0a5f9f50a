"""Build ``libconv_im2win.so`` in-tree with hipcc for gfx950.

Usage: ``python -m cnn_convolution_im2win_amd.build`` (or ``build()``).
Every source compiles to an object in ``_build/`` in parallel, then the
objects link into ``cnn_convolution_im2win_amd/libconv_im2win.so``.
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libconv_im2win.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "transform.hip", "conv_fp32.hip", "conv_fp32_mfma.hip", "conv_mfma.hip", "conv_mfma_f16.hip",
           "conv_mfma_bf16.hip", "conv_dw.hip", "conv_dw_implicit.hip", "conv_implicit.hip", "conv_implicit_f16.hip",
           "conv_implicit_bf16.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-I", INCLUDE, "-I", CSRC,
    # packed-fp32 VALU instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + CFLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # the host pass warns that it does not know the packed-fp32 feature; drop that
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l and l.strip()]
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library; returns its path."""
    if not shutil.which(HIPCC) and not os.path.exists(HIPCC):
        raise RuntimeError("hipcc not found")
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)

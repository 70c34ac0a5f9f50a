"""Build ``libconv_im2win.so`` in-tree with hipcc for gfx950.

Usage: ``python -m cnn_convolution_im2win_amd.build`` (or ``build()``).
Every source compiles to an object in ``_build/`` in parallel, then the
objects link into ``cnn_convolution_im2win_amd/libconv_im2win.so``.

``build_variants()`` also links the ablation variants: copies of the library
in which one kernel is compiled with some of its optimizations switched off
(the im2win paper, §IV-E, ablates its tensor-core kernel the same way).
Each lands in ``variants/<name>/libconv_im2win.so`` next to this file; only
the switched kernel's sources are recompiled, the other objects are the main
build's (every kernel lives in an anonymous namespace, so objects built with
different switches link together).
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

SOURCES = ["api.cpp", "transform.hip", "conv_fp32.hip", "conv_fp32_mfma.hip", "conv_fp32_m16.hip", "conv_mfma.hip", "conv_mfma_f16.hip",
           "conv_mfma_bf16.hip", "conv_dw.hip", "conv_dw_implicit.hip", "conv_implicit.hip", "conv_implicit_f16.hip",
           "conv_implicit_bf16.hip", "conv_band_f16.hip", "conv_band_bf16.hip", "conv_narrow.hip",
           "conv_narrow_f16.hip", "conv_narrow_bf16.hip"]

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


# name -> (compile definitions, sources recompiled with them, what it measures).
# The row-kernel variants are built for the fp16 3x3 64 -> 64 layer they are
# timed and checked on (CIW_ROWS_ABLATION_ONLY: other row-kernel plans are
# turned down with an error), which keeps their builds short.
VARIANTS = {
    # the materialised-window row kernel (conv_mfma_rows_kernel), fp16 inputs
    "rows_baseline": (["-DCIW_ROWS_ABLATION_ONLY=1"], ["conv_mfma.hip", "conv_mfma_f16.hip"],
                      "row kernel as in the library"),
    "rows_no_double": (["-DCIW_ROWS_ABLATION_ONLY=1", "-DCIW_ABLATE_ROWS_NO_DOUBLE=1"], ["conv_mfma.hip", "conv_mfma_f16.hip"],
                       "one row buffer: each row copied when it is multiplied, then waited for"),
    "rows_no_async": (["-DCIW_ROWS_ABLATION_ONLY=1", "-DCIW_ABLATE_ROWS_NO_ASYNC=1"], ["conv_mfma.hip", "conv_mfma_f16.hip"],
                      "rows copied global -> registers -> LDS"),
    "rows_no_pad": (["-DCIW_ROWS_ABLATION_ONLY=1", "-DCIW_ABLATE_ROWS_NO_PAD=1"], ["conv_mfma.hip", "conv_mfma_f16.hip"],
                    "no LDS pad chunks: a fragment's lanes read the same banks"),
    "rows_no_index": (["-DCIW_ROWS_ABLATION_ONLY=1", "-DCIW_ABLATE_ROWS_NO_INDEX=1"], ["conv_mfma.hip", "conv_mfma_f16.hip"],
                      "plain divisions and no filter re-layout: fragments gathered in the kernel"),
    # the window-row buffers of the in-LDS kernel (conv_mfma_implicit_kernel)
    # (CIW_BAND_OFF keeps these on that kernel where the band kernel would run)
    "implicit_baseline": (["-DCIW_BAND_OFF=1"], ["conv_implicit.hip", "conv_implicit_f16.hip"],
                          "row-band in-LDS window kernel as in the library"),
    "implicit_no_double": (["-DCIW_BAND_OFF=1", "-DCIW_ABLATE_NO_DOUBLE=1"],
                           ["conv_implicit.hip", "conv_implicit_f16.hip"],
                           "input row copied at the step that needs it, then waited for"),
    "implicit_no_async": (["-DCIW_BAND_OFF=1", "-DCIW_ABLATE_NO_ASYNC=1"],
                          ["conv_implicit.hip", "conv_implicit_f16.hip"],
                          "rows copied global -> registers -> LDS"),
    "implicit_no_xcd": (["-DCIW_BAND_OFF=1", "-DCIW_ABLATE_NO_XCD=1"],
                        ["conv_implicit.hip", "conv_implicit_f16.hip"],
                        "bands in dispatch order"),
}
VARIANT_DIR = os.path.join(PKG, "variants")


def variant_path(name: str) -> str:
    return os.path.join(VARIANT_DIR, name, "libconv_im2win.so")


def build_variants(verbose: bool = False) -> None:
    """Link every ablation variant (needs the main build's objects)."""
    main_objs = {s: os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES}
    missing = [o for o in main_objs.values() if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"build the library first (missing {missing[0]})")
    jobs = []
    for name, (defs, srcs, _) in VARIANTS.items():
        for src in srcs:
            jobs.append((name, defs, src))

    def one(job):
        name, defs, src = job
        bdir = os.path.join(BUILD_DIR, "variants", name)
        os.makedirs(bdir, exist_ok=True)
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC] + CFLAGS + defs + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"{name}: hipcc failed for {src}:\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(one, jobs))
    for name, (defs, srcs, _) in VARIANTS.items():
        bdir = os.path.join(BUILD_DIR, "variants", name)
        objs = [os.path.join(bdir, os.path.splitext(s)[0] + ".o") if s in srcs else main_objs[s]
                for s in SOURCES]
        out = variant_path(name)
        os.makedirs(os.path.dirname(out), exist_ok=True)
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out + ".tmp"] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"{name}: link failed:\n{r.stderr}")
        os.replace(out + ".tmp", out)
        if verbose:
            print(f"built {out}")


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
    if "--variants" in sys.argv:
        build_variants(verbose=True)

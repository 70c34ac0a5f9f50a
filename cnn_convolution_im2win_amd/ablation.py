"""Ablation of the in-LDS fp16/bf16 window kernel on MI355X.

The im2win paper (§IV-E) measures its tensor-core kernel without double
buffering, without asynchronous copies and without its zig-zag order.  The
MI355X counterparts are compile-time switches of conv_mfma_implicit_kernel
(csrc/conv_implicit_impl.hpp):

  no_double  input rows copied at the step that needs them, then waited for
  no_async   rows copied global memory -> registers -> LDS, not straight to LDS
  no_xcd     bands in dispatch order, not placed XCD by XCD

Usage, from the repository root:
  python -m cnn_convolution_im2win_amd.ablation --build   # after the main build; CPU is enough
  python -m cnn_convolution_im2win_amd.ablation --run     # on a GPU: parity check + timing per variant

Each variant is a full copy of the library with the switch set; --run
checks every variant's output on the 128x64x56x56 fp16 layer against the
CPU oracle at sampled points before timing it (five runs of 50 calls back
to back after 10 warm-ups, HIP events around each run; the median run),
each in its own process, and prints one JSON line.
"""
from __future__ import annotations

import json
import os
import subprocess
import sys

from . import build as _build

VARIANTS = {
    "baseline": [],
    "no_double": ["-DCIW_ABLATE_NO_DOUBLE=1"],
    "no_async": ["-DCIW_ABLATE_NO_ASYNC=1"],
    "no_xcd": ["-DCIW_ABLATE_NO_XCD=1"],
    "none": ["-DCIW_ABLATE_NO_DOUBLE=1", "-DCIW_ABLATE_NO_ASYNC=1", "-DCIW_ABLATE_NO_XCD=1"],
}
VARIANT_SOURCES = ["conv_implicit.hip", "conv_implicit_f16.hip", "conv_implicit_bf16.hip"]
OUT_DIR = os.path.join(_build.PKG, "ablation")


def lib_path(name: str) -> str:
    return os.path.join(OUT_DIR, name, "libconv_im2win.so")


def build_variants() -> None:
    """Compile the kernel's sources once per variant and link each with the
    main build's other objects."""
    from concurrent.futures import ThreadPoolExecutor
    others = [os.path.join(_build.BUILD_DIR, os.path.splitext(s)[0] + ".o")
              for s in _build.SOURCES if s not in VARIANT_SOURCES]
    missing = [o for o in others if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"build the library first (missing {missing[0]})")

    def one(item):
        name, flags = item
        bdir = os.path.join(_build.BUILD_DIR, "ablation", name)
        os.makedirs(bdir, exist_ok=True)
        objs = []
        for src in VARIANT_SOURCES:
            obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
            cmd = [_build.HIPCC] + _build.CFLAGS + flags + ["-x", "hip", "-c",
                                                           os.path.join(_build.CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"{name}: {src} failed:\n{r.stderr}")
            objs.append(obj)
        out = lib_path(name)
        os.makedirs(os.path.dirname(out), exist_ok=True)
        cmd = [_build.HIPCC, f"--offload-arch={_build.ARCH}", "-shared", "-fPIC", "-o", out] + others + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"{name}: link failed:\n{r.stderr}")
        return out

    with ThreadPoolExecutor(max_workers=len(VARIANTS)) as ex:
        for out in ex.map(one, VARIANTS.items()):
            print(f"built {out}", flush=True)


def time_variant(name: str) -> dict:
    """Parity check and timing of one variant (in this process)."""
    import numpy as np
    import torch
    from . import _lib
    _lib.LIB_PATH = lib_path(name)
    import cnn_convolution_im2win_amd as ciw
    root = os.path.dirname(_build.PKG)
    if root not in sys.path:
        sys.path.insert(0, root)
    import oracle
    import workloads

    L = workloads.LAYERS["resnet_3x3_fp16"]
    x, w, _ = workloads.make_inputs(L)
    xd = torch.from_numpy(x).to("cuda")
    wd = torch.from_numpy(w).to("cuda")
    desc = ciw.make_desc(L.x_shape, L.w_shape, L.stride, L.pad, L.dil, 1)
    y = torch.empty((L.N, L.K, 56, 56), dtype=torch.float16, device="cuda")
    nbytes = ciw.conv2d_implicit_workspace_bytes(desc, ciw.CIW_F16, ciw.CIW_F16, 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def call():
        ciw.conv2d_fwd(xd, wd, None, y, ws, L.stride, L.pad, L.dil, flags=ciw.CIW_FLAG_IMPLICIT)

    call()
    torch.cuda.synchronize()
    got = y.float().cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(5)
    idx = np.stack([rng.integers(0, s, 800) for s in got.shape], axis=1)
    ref = oracle.conv2d_points(x.astype(np.float64), w.astype(np.float64), None, idx, L.stride,
                               L.pad, L.dil, 1)
    err = float(np.max(np.abs(got[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]] - ref)) /
                np.max(np.abs(ref)))
    if not err <= 2e-2:
        raise AssertionError(f"{name}: rel err {err} > 2e-2")
    for _ in range(10):
        call()
    torch.cuda.synchronize()
    # events only around runs of calls: one recorded between calls costs
    # GPU time of its own
    ms = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(50):
            call()
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b) / 50)
    ms.sort()
    flops = 2 * L.N * L.K * L.C * L.R * L.S * 56 * 56
    med = ms[len(ms) // 2]
    return {"variant": name, "median_us": round(med * 1e3, 2), "best_us": round(ms[0] * 1e3, 2),
            "tflops": round(flops / (med * 1e-3) / 1e12, 1), "rel_err": err}


def run_all() -> dict:
    res = {}
    for name in VARIANTS:
        if not os.path.exists(lib_path(name)):
            raise RuntimeError(f"{lib_path(name)} missing: run --build first")
        r = subprocess.run([sys.executable, "-m", "cnn_convolution_im2win_amd.ablation", "--time", name],
                           capture_output=True, text=True, timeout=300)
        if r.returncode != 0:
            raise RuntimeError(f"{name} failed:\n{r.stdout}\n{r.stderr}")
        res[name] = json.loads(r.stdout.strip().splitlines()[-1])
        print(f"# {json.dumps(res[name])}", file=sys.stderr, flush=True)
    base = res["baseline"]["median_us"]
    for v in res.values():
        v["vs_baseline"] = round(v["median_us"] / base, 3)
    return res


if __name__ == "__main__":
    if "--build" in sys.argv:
        build_variants()
    elif "--time" in sys.argv:
        print(json.dumps(time_variant(sys.argv[sys.argv.index("--time") + 1])), flush=True)
    elif "--run" in sys.argv:
        print(json.dumps({"layer": "resnet_3x3_fp16 (128x64x56x56 -> 64, 3x3, fp16), CIW_FLAG_IMPLICIT",
                          "variants": run_all()}), flush=True)
    else:
        print(__doc__)

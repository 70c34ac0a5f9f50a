#!/usr/bin/env python3
"""Benchmark of the im2win forward convolution on one MI355X.

One step = the whole hot path over one batch of synthetic input, through the
C ABI on one HIP stream: the im2win repack (conv_im2win_transform) and the
windowed contraction with its bias epilogue (conv2d_fwd / conv2d_dw_fwd on the
ready window tensor).  Inputs are resident in HBM before timing starts.

Prints ONE JSON line.  `value` is the TFLOP/s of the headline layer's step
(2*N*K*(C/G)*R*S*P*Q per second; with the fused pool, P and Q count only the
pixels its 2x2 regions cover), K steps back to back between two device
synchronisations.  `roofline` is the headline contraction's position: call
level (HIP events on its stream around back-to-back calls) with the dominant
kernel's own traced duration beside it (`kernel_only`).  `layers` holds
every layer of the set, each with
  - the step, back to back (events and wall clock) and traced call by call:
    best and median over --iters calls, warm (back to back) and cold (a
    read of 1 GiB before each call evicts the L2 caches and the 256 MB
    Infinity Cache), per kernel, kernel sum and call span;
  - the repack and the contraction on their own, and the in-LDS call
    (CIW_FLAG_IMPLICIT) where the library runs the layer that way, each
    with its roofline (the compute unit is the one the traced kernels run
    on, so the bound follows the library's own choice);
  - the CPU oracle on a bounded sample and the speedup over it (the
    headline layer also gets the numpy im2col point);
  - the memory table: peak device memory and time of one call per
    processing strategy (whole batch, 16-image chunks, single images, the
    in-LDS call; the im2col matrix size; MIOpen with --miopen).

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--iters I]
                  [--headline-only] [--epilogue none|relu|relu_pool]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "conv2d fwd TFLOP/s (2NKCRSPQ/s) and % of MI355X MFMA/HBM roofline"

# MI355X published peaks (dense)
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"mfma_f16": 2516.6, "mfma_bf16": 2516.6, "valu_f32": 157.3}
# The OpenCL-Benchmarks page times exactly the 1x512x13x13 -> 1024 3x3 layer
# (direct convolution, Mali T860): 913.301 ms run time.  Context only.
PAGE_BASELINE = {"mid_3x3_fp32": 2 * 1024 * 512 * 9 * 169 / 913.301e-3 / 1e12}

DEFAULT_WORKLOAD = "mid_3x3_fp32"
EPILOGUES = ("none", "relu", "relu_pool")


def describe(L: workloads.Layer) -> str:
    return (f"{L.name}: N={L.N} C={L.C} H={L.H} W={L.W} K={L.K} {L.R}x{L.S} "
            f"stride={L.stride[0]} pad={L.pad[0]} groups={L.groups} {L.dtype}->{L.out_dtype}"
            f"{' bias' if L.b_dist is not None else ''}")


class Step:
    """Pre-marshalled C-ABI calls for one layer (argument marshalling happens
    once, outside the timed region)."""

    def __init__(self, L: workloads.Layer, epilogue: str = "none"):
        import numpy as np  # noqa: F401
        import torch
        import cnn_convolution_im2win_amd as ciw
        from cnn_convolution_im2win_amd import _lib

        self.L = L
        self.epilogue = epilogue
        self.ciw = ciw
        self.epi_flags = {"none": 0, "relu": ciw.CIW_FLAG_RELU,
                          "relu_pool": ciw.CIW_FLAG_RELU | ciw.CIW_FLAG_MAXPOOL2}[epilogue]
        self.lib = _lib.load()
        code = {"f32": ciw.CIW_F32, "f16": ciw.CIW_F16, "bf16": ciw.CIW_BF16}
        self.in_code, self.out_code = code[L.dtype], code[L.out_dtype]
        x, w, b = workloads.make_inputs(L)

        def dev(a):
            if a is None:
                return None
            t = torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if L.dtype == "bf16" else a))
            t = t.to("cuda")
            return t.view(torch.bfloat16) if L.dtype == "bf16" else t

        self.x, self.w, self.b = dev(x), dev(w), dev(b)
        self.desc = ciw.make_desc(L.x_shape, L.w_shape, L.stride, L.pad, L.dil, L.groups)
        self.depthwise = L.groups > 1
        self.layout = ciw.CIW_WIN_HWC if (L.dtype != "f32" and not self.depthwise) else ciw.CIW_WIN_CHW
        self.P, self.Q = ciw.conv_im2win_output_dims(self.desc)
        Po, Qo = ciw.conv2d_output_dims(self.desc, self.epi_flags)
        tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
        self.y = torch.empty((L.N, L.K, Po, Qo), dtype=tdt[L.out_dtype], device="cuda")
        self.ws_bytes = ciw.conv2d_workspace_bytes(self.desc, self.in_code, L.N)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")
        self.win_bytes = ciw.conv_im2win_window_bytes(self.desc, self.in_code, self.layout, L.N)
        # one side stream for everything the step launches
        self.stream = torch.cuda.Stream()
        self.sp = self.stream.cuda_stream
        self.fn = self.lib.conv2d_dw_fwd if self.depthwise else self.lib.conv2d_fwd
        self.dref = ctypes.byref(self.desc)
        self.args_fwd = (self.dref, self.in_code, self.out_code, None, self.w.data_ptr(),
                         None if self.b is None else self.b.data_ptr(), self.y.data_ptr(),
                         self.ws.data_ptr(), self.ws_bytes,
                         ciw.CIW_FLAG_WINDOW_READY | self.epi_flags, self.sp)
        self.args_tr = (self.dref, self.in_code, self.layout, self.x.data_ptr(),
                        self.ws.data_ptr(), self.sp)

    def transform(self):
        st = self.lib.conv_im2win_transform(*self.args_tr)
        if st != 0:
            raise RuntimeError(f"conv_im2win_transform: status {st}")

    def contract(self):
        st = self.fn(*self.args_fwd)
        if st != 0:
            raise RuntimeError(f"conv2d_fwd: status {st}")

    # ---- algorithmic work
    def flops(self) -> int:
        # with the pool, only the pixels of the 2x2 regions reach an output
        L = self.L
        P, Q = self.P, self.Q
        if self.epilogue == "relu_pool":
            P, Q = 2 * (P // 2), 2 * (Q // 2)
        return 2 * L.N * L.K * (L.C // L.groups) * L.R * L.S * P * Q

    def bytes_x(self):
        return self.x.numel() * self.x.element_size()

    def bytes_w(self):
        return self.w.numel() * self.w.element_size()

    def bytes_b(self):
        return 0 if self.b is None else self.b.numel() * self.b.element_size()

    def bytes_y(self):
        return self.y.numel() * self.y.element_size()

    def contraction_bytes(self):
        # window tensor read once, filters and bias once, output (pooled, if
        # the pool is fused) written once
        return self.win_bytes + self.bytes_w() + self.bytes_b() + self.bytes_y()

    def transform_bytes(self):
        return self.bytes_x() + self.win_bytes

    def contraction_roofline(self, kernel_ms: float) -> dict:
        """Roofline position of the contraction kernel: compute-bound when its
        arithmetic intensity is above the ridge, else bound by HBM."""
        L = self.L
        if self.depthwise:
            peak_c, unit_c = PEAK_TFLOPS["valu_f32"], "alu"
        elif L.dtype == "f32":
            peak_c, unit_c = PEAK_TFLOPS["valu_f32"], "alu"
        else:
            peak_c, unit_c = PEAK_TFLOPS["mfma_" + L.dtype], "mfma"
        ai = self.flops() / self.contraction_bytes()
        ridge = peak_c * 1e12 / (PEAK_HBM_GBS * 1e9)
        s = kernel_ms * 1e-3
        if ai >= ridge:
            ach = self.flops() / s / 1e12
            return {"bound": unit_c, "achieved": round(ach, 3), "peak": peak_c,
                    "unit": "TFLOP/s", "frac": round(ach / peak_c, 4), "traffic": None}
        ach = self.contraction_bytes() / s / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None}


def kernel_source_hash() -> str:
    """sha256 over the HIP/C++ sources of the library (which kernels the
    stored counter readings belong to)."""
    import hashlib
    csrc = os.path.join(ROOT, "cnn_convolution_im2win_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".cpp", ".hpp")):
            h.update(name.encode())
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def traffic_key(L: workloads.Layer, epilogue: str) -> str:
    return L.name if epilogue == "none" else f"{L.name}+{epilogue}"


def stored_traffic(workload: str):
    """HBM bytes per contraction call from profiles/traffic.json (rocprofv3
    FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's reading), or None when
    the file is missing or was measured on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    if data.get("source_sha256") != kernel_source_hash():
        return None
    entry = data.get("workloads", {}).get(workload)
    return None if entry is None else entry.get("bytes_per_call")


SETTLE_S = 0.5   # untimed back-to-back calls before a layer's first timed loop (--settle)


def settle(fn, seconds: float = None):
    """Call fn back to back for about `seconds` (untimed): the GPU's clocks
    ramp up under load over a few hundred milliseconds, and a timed loop of
    a few dozen 30 us steps started from idle would measure the ramp."""
    import torch
    t_end = time.perf_counter() + (SETTLE_S if seconds is None else min(seconds, SETTLE_S))
    while time.perf_counter() < t_end:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()


def loop_ms(stream, fn, steps: int, warmup: int):
    """Mean time per iteration of `fn` over `steps` back-to-back iterations:
    HIP events recorded on `stream` just before the first and just after
    the last (the GPU's time), and the host's wall clock between two device
    synchronisations (the figure throughput is quoted on).  Events between
    iterations are left out on purpose: each one recorded on a stream costs
    about 3-4 us of GPU time on this GPU, as much as a small kernel."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return e0.elapsed_time(e1) / steps, wall


CALL_REPS = 5   # repetitions of a per-call loop; the median is reported


def call_ms(stream, fn, steps: int, warmup: int, reps: int = CALL_REPS):
    """Per-call time of `fn`: `reps` runs of `loop_ms` (K calls back to back
    between two HIP events), returning (median, best) of the runs' means, so
    that one slow burst on a shared box does not decide the figure."""
    runs = sorted(loop_ms(stream, fn, steps, warmup if i == 0 else 1)[0] for i in range(reps))
    return runs[len(runs) // 2], runs[0]


def time_steps(step: Step, steps: int, warmup: int):
    """K timed steps, each the two C-ABI calls on the step's stream,
    bracketed by a device synchronisation on both sides (wall clock) and by
    one pair of HIP events on that stream.  Then each call on its own: K
    transform calls back to back, and K contraction calls back to back on the
    window tensor the last transform left (HIP events around each loop; the
    median of CALL_REPS such loops).  (Replaying the calls as HIP graphs was measured
    slower here than launching them directly, so the step launches them
    directly.)"""
    def one():
        step.transform()
        step.contract()
    settle(one)
    gpu_ms, wall_ms = loop_ms(step.stream, one, steps, warmup)
    tr_ms, _ = call_ms(step.stream, step.transform, steps, 2)
    co_ms, _ = call_ms(step.stream, step.contract, steps, 2)
    return wall_ms, gpu_ms, tr_ms, co_ms


def cpu_baseline(L: workloads.Layer, seconds: float) -> dict:
    """The CPU oracle (fp64 direct convolution, OpenMP over (n, k)) on a
    bounded sample of the layer: whole images, as many as fit ~`seconds`."""
    import numpy as np
    import oracle
    x, w, b = workloads.make_inputs(L)
    f = lambda a: None if a is None else workloads.to_f64(a, L.dtype)
    x, w, b = f(x), f(w), f(b)
    P, Q = oracle.out_dims(L.x_shape, L.w_shape, L.stride, L.pad, L.dil, L.groups)
    flops_img = 2 * L.K * (L.C // L.groups) * L.R * L.S * P * Q
    t0 = time.perf_counter()
    oracle.conv2d(x[:1], w, b, L.stride, L.pad, L.dil, L.groups)
    one = time.perf_counter() - t0
    reps, n_img = 1, 1
    if one < seconds:
        want = max(1, int(seconds / max(one, 1e-6)))
        n_img = min(L.N, want)
        reps = max(1, want // n_img)
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.conv2d(x[:n_img], w, b, L.stride, L.pad, L.dil, L.groups)
    dt = time.perf_counter() - t0
    tflops = flops_img * n_img * reps / dt / 1e12
    return {"value": round(tflops, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{n_img} of {L.N} images x {reps} repeats ({dt:.1f} s wall); "
                      f"fp64 seven-loop direct convolution"}


def time_unfused(L: workloads.Layer, epilogue: str, steps: int, warmup: int) -> float:
    """Context for a fused epilogue: mean ms of the plain contraction followed
    by torch's ReLU (and 2x2 max-pool) over the full output, on one stream."""
    import torch
    import torch.nn.functional as F
    step = Step(L)

    def run():
        step.contract()
        with torch.cuda.stream(step.stream):
            y = torch.relu(step.y)
            if epilogue == "relu_pool":
                y = F.max_pool2d(y, 2)
        return y

    step.transform()
    ms, _ = loop_ms(step.stream, run, steps, warmup)
    return ms


def memory_report(L: workloads.Layer, steps: int = 5, miopen: bool = False,
                  epilogue: str = "none") -> dict:
    """Peak device memory and time per call of each processing strategy.

    The library allocates nothing: a call's footprint is x, w, b and y plus
    the workspace, whose size follows from how many images one chunk
    repacks (conv2d_workspace_bytes).  Peaks are read from torch's caching
    allocator around a fresh allocation of every buffer."""
    import numpy as np
    import torch
    import torch.nn.functional as F
    import cnn_convolution_im2win_amd as ciw

    code = {"f32": ciw.CIW_F32, "f16": ciw.CIW_F16, "bf16": ciw.CIW_BF16}[L.dtype]
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
    x, w, b = workloads.make_inputs(L)

    def dev(a):
        if a is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if L.dtype == "bf16" else a))
        t = t.to("cuda")
        return t.view(torch.bfloat16) if L.dtype == "bf16" else t

    desc = ciw.make_desc(L.x_shape, L.w_shape, L.stride, L.pad, L.dil, L.groups)
    P, Q = ciw.conv_im2win_output_dims(desc)
    eb = workloads.ELEM_BYTES[L.dtype]
    io_bytes = (L.N * L.C * L.H * L.W + L.K * (L.C // L.groups) * L.R * L.S
                + (L.K if L.b_dist is not None else 0)) * eb + \
        L.N * L.K * P * Q * workloads.ELEM_BYTES[L.out_dtype]

    def peak_and_time(run_once):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        state = run_once(None)                 # allocates every buffer, runs once
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            run_once(state)
        e1.record()
        torch.cuda.synchronize()
        del state
        return peak, e0.elapsed_time(e1) / steps

    def im2win(n_chunk):
        ws_bytes = ciw.conv2d_workspace_bytes(desc, code, n_chunk)

        def run_once(state):
            if state is None:
                xd, wd, bd = dev(x), dev(w), dev(b)
                y = torch.empty((L.N, L.K, P, Q), dtype=tdt[L.out_dtype], device="cuda")
                ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
                state = (xd, wd, bd, y, ws)
            xd, wd, bd, y, ws = state
            fn = ciw.conv2d_dw_fwd if L.groups > 1 else ciw.conv2d_fwd
            fn(xd, wd, bd, y, ws, L.stride, L.pad, L.dil)
            return state

        peak, ms = peak_and_time(run_once)
        return {"chunk_images": n_chunk, "workspace_bytes": ws_bytes, "peak_bytes": peak,
                "ms": round(ms, 4)}

    out = {"inputs_outputs_bytes": io_bytes}
    for tag, n in (("im2win_full_batch", L.N), ("im2win_chunk16", min(L.N, 16)),
                   ("im2win_single_image", 1)):
        if tag != "im2win_full_batch" and n == L.N:
            continue
        out[tag] = im2win(n)
    per_image = (L.C // L.groups) * L.groups * L.R * L.S * P * Q * eb
    out["im2col_matrix_bytes"] = {"single_image": per_image, "full_batch": per_image * L.N}

    def miopen_run(state):
        if state is None:
            state = (dev(x), dev(w), dev(b))
        xd, wd, bd = state
        F.conv2d(xd, wd, bd, L.stride, L.pad, L.dil, L.groups)
        return state

    # the in-LDS call: no window tensor, the workspace (if any) holds only the
    # re-laid-out filter
    flags = ciw.CIW_FLAG_IMPLICIT
    out_code = {"f32": ciw.CIW_F32, "f16": ciw.CIW_F16, "bf16": ciw.CIW_BF16}[L.out_dtype]
    try:
        imp_bytes = ciw.conv2d_implicit_workspace_bytes(desc, code, out_code, flags)
    except ciw.Im2winError:
        imp_bytes = None
    if imp_bytes is not None:
        def run_imp(state):
            if state is None:
                xd, wd, bd = dev(x), dev(w), dev(b)
                y = torch.empty((L.N, L.K, P, Q), dtype=tdt[L.out_dtype], device="cuda")
                ws = torch.empty(max(imp_bytes, 16), dtype=torch.uint8, device="cuda")
                state = (xd, wd, bd, y, ws)
            xd, wd, bd, y, ws = state
            fn = ciw.conv2d_dw_fwd if L.groups > 1 else ciw.conv2d_fwd
            fn(xd, wd, bd, y, ws, L.stride, L.pad, L.dil, flags=flags)
            return state
        peak, ms = peak_and_time(run_imp)
        out["in_lds"] = {"workspace_bytes": imp_bytes, "peak_bytes": peak, "ms": round(ms, 4)}
    if miopen:
        try:
            peak, ms = peak_and_time(miopen_run)
            out["miopen_conv2d"] = {"peak_bytes": peak, "ms": round(ms, 4)}
        except Exception as e:   # context only
            out["miopen_conv2d"] = {"error": str(e)[:200]}
    return out


def time_fp32_kernels(step: Step, steps: int, warmup: int):
    """The fp32 contraction (window ready) with each kernel forced: matrix
    cores (CIW_FLAG_FP32_MFMA) and vector ALUs (CIW_FLAG_FP32_VALU), K calls
    back to back each, HIP events around the loop; the automatic choice is
    the step's own contraction.  None for layers the matrix-core kernel does
    not run."""
    import torch
    ciw = step.ciw
    L = step.L
    if L.dtype != "f32" or step.depthwise or step.epilogue == "relu_pool" or \
            L.R != L.S or L.R not in (1, 3) or step.Q > 192:
        return None
    step.transform()
    out = {}
    for name, flag in (("matrix", ciw.CIW_FLAG_FP32_MFMA), ("vector", ciw.CIW_FLAG_FP32_VALU)):
        args = list(step.args_fwd)
        args[9] = args[9] | flag

        def call():
            st = step.fn(*args)
            if st != 0:
                raise RuntimeError(f"conv2d_fwd ({name}): status {st}")
        settle(call, 0.2)
        ms, _ = call_ms(step.stream, call, steps, warmup)
        out[name] = {"contract_ms": round(ms, 5),
                     "contract_tflops": round(step.flops() / (ms * 1e-3) / 1e12, 3)}
    return out


# ---------------------------------------------------------------- kernel traces
def is_library_kernel(name: str) -> bool:
    """Whether a traced kernel is one of this library's (namespace ciw),
    whether the tracer reports its name mangled or demangled."""
    return name.startswith("_ZN3ciw") or "ciw::" in name


def short_name(name: str) -> str:
    """Readable name of one of this library's kernels from its symbol,
    mangled or demangled: the function's identifier, without namespaces,
    template arguments or parameters."""
    s = name
    if s.startswith("_ZN3ciw"):
        s = s[len("_ZN3ciw"):]
        if s.startswith("12_GLOBAL__N_1"):
            s = s[len("12_GLOBAL__N_1"):]
        i = 0
        while i < len(s) and s[i].isdigit():
            i += 1
        if i:
            n = int(s[:i])
            return s[i:i + n]
    if "ciw::" in s:
        s = s[s.index("ciw::"):].replace("(anonymous namespace)", "anon")
        cut = len(s)
        for j, ch in enumerate(s):       # the qualified name ends at the first '<' or '('
            if ch in "<(":
                cut = j
                break
        s = s[:cut]
        return s.split("::")[-1]
    return s.split("(")[0][:60]


def kernel_trace(stream, fn, iters: int, flush=None):
    """`iters` calls of fn on `stream` under torch's profiler (the GPU's own
    kernel timestamps); with `flush` (a >= 512 MB device buffer) each call is
    preceded, on the same stream, by a read of that whole buffer (a sum),
    which evicts the L2 caches and the 256 MB Infinity Cache and leaves
    them holding clean lines (the cold regime: a write would leave dirty
    lines that the measured call would have to write back).  Returns one
    list per call of (kernel, start_us, duration_us) for this library's
    kernels, in launch order."""
    import torch
    from torch.profiler import ProfilerActivity, profile
    fn()
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        for i in range(iters):
            if flush is not None:
                with torch.cuda.stream(stream):
                    flush.view(torch.int32).sum()
            fn()
        torch.cuda.synchronize()
    evs = [e for e in prof.events()
           if e.device_type.name == "CUDA" and is_library_kernel(str(e.name))]
    evs.sort(key=lambda e: e.time_range.start)
    if not evs or len(evs) % iters:
        raise RuntimeError(f"trace holds {len(evs)} library kernels for {iters} calls")
    k = len(evs) // iters
    return [[(short_name(e.name), e.time_range.start, e.time_range.end - e.time_range.start)
             for e in evs[i * k:(i + 1) * k]] for i in range(iters)]


def trace_stats(calls) -> dict:
    """Best and median over the calls of: each kernel's duration, the sum of
    the kernels' durations, and the call's span (first kernel's start to the
    last one's end, launch gaps included); microseconds."""
    import statistics

    def bm(v):
        return {"best_us": round(min(v), 2), "median_us": round(statistics.median(v), 2)}
    names = [n for n, _, _ in calls[0]]
    out = {"calls": len(calls), "kernels": {}}
    for j, n in enumerate(names):
        key = n if names.count(n) == 1 else f"{n}#{j}"
        out["kernels"][key] = bm([c[j][2] for c in calls])
    out["kernel_sum"] = bm([sum(d for _, _, d in c) for c in calls])
    out["span"] = bm([c[-1][1] + c[-1][2] - c[0][1] for c in calls])
    dom = max(range(len(names)), key=lambda j: statistics.median(c[j][2] for c in calls))
    out["dominant"] = names[dom]
    out["dominant_us"] = bm([c[dom][2] for c in calls])
    return out


def roofline_entry(flops: int, nbytes: int, dtype: str, dominant: str, ms: float) -> dict:
    """Roofline position of a call or kernel lasting `ms`: the compute peak is
    that of the unit the library's dominant kernel runs on (named by the
    trace: the matrix cores for the 'mfma' kernels, the vector ALUs for the
    fp32 VALU kernels), HBM for layers below that unit's ridge point and for
    depthwise; both fractions are given, `frac` is the one of the bound."""
    if "mfma" in dominant and dtype in ("f16", "bf16"):
        unit, peak = "mfma", PEAK_TFLOPS["mfma_" + dtype]
    elif "mfma" in dominant:
        unit, peak = "mfma", PEAK_TFLOPS["valu_f32"]   # fp32 MFMA: 157.3 TFLOP/s dense
    else:
        unit, peak = "alu", PEAK_TFLOPS["valu_f32"]
    s = ms * 1e-3
    tf = flops / s / 1e12
    gbs = nbytes / s / 1e9
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    hbm_bound = dominant.startswith("conv_dw") or flops / nbytes < ridge
    out = {"bound": "hbm" if hbm_bound else unit,
           "achieved": round(gbs, 1) if hbm_bound else round(tf, 3),
           "peak": PEAK_HBM_GBS if hbm_bound else peak,
           "unit": "GB/s" if hbm_bound else "TFLOP/s",
           "frac": round((gbs / PEAK_HBM_GBS) if hbm_bound else (tf / peak), 4),
           "compute_frac": round(tf / peak, 4), "compute_unit": unit,
           "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
           "algorithmic_bytes": nbytes, "flops": flops}
    return out


def implicit_call(step: "Step"):
    """The in-LDS conv2d_fwd call (CIW_FLAG_IMPLICIT: window rows built in
    LDS from x) for the step's layer, or None when the library does not run
    the layer that way."""
    import torch
    ciw = step.ciw
    flags = ciw.CIW_FLAG_IMPLICIT | step.epi_flags
    try:
        nbytes = ciw.conv2d_implicit_workspace_bytes(step.desc, step.in_code, step.out_code, flags)
    except ciw.Im2winError:
        return None, 0
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    args = (step.dref, step.in_code, step.out_code, step.x.data_ptr(), step.w.data_ptr(),
            None if step.b is None else step.b.data_ptr(), step.y.data_ptr(), ws.data_ptr(),
            nbytes, flags, step.sp)

    def call(_ws=ws):
        st = step.fn(*args)
        if st != 0:
            raise RuntimeError(f"conv2d_fwd (in-LDS): status {st}")
    return call, nbytes


def measure_layer2(L: workloads.Layer, steps: int, warmup: int, iters: int, flush,
                   epilogue: str = "none", trace: bool = True, unfused: bool = True) -> tuple:
    """Every measurement of one layer: the step (repack + contraction) timed
    back to back with HIP events and the wall clock; warm and cold kernel
    traces of the step, of the contraction call and of the in-LDS call; the
    roofline of each call (call level: HIP events around back-to-back calls;
    kernel level: the dominant kernel's traced duration)."""
    step = Step(L, epilogue)
    wall_ms, gpu_ms, tr_ms, co_ms = time_steps(step, steps, warmup)
    fl = step.flops()
    res = {"layer": describe(L), "flops": fl,
           "step": {"ms": round(wall_ms, 5), "gpu_ms": round(gpu_ms, 5),
                    "tflops": round(fl / (wall_ms * 1e-3) / 1e12, 3),
                    "calls": "conv_im2win_transform + conv2d_fwd(window ready)"}}

    def one():
        step.transform()
        step.contract()
    if trace:
        tw = trace_stats(kernel_trace(step.stream, one, iters))
        tc = trace_stats(kernel_trace(step.stream, one, iters, flush))
        res["step"]["warm"] = tw
        res["step"]["cold"] = tc
        res["step"]["tflops_best_warm"] = round(fl / (tw["span"]["best_us"] * 1e-6) / 1e12, 3)
        res["step"]["tflops_best_cold"] = round(fl / (tc["span"]["best_us"] * 1e-6) / 1e12, 3)

    # the repack on its own
    t_tr = trace_stats(kernel_trace(step.stream, step.transform, iters)) if trace else None
    res["transform"] = {"call_ms": round(tr_ms, 5), "warm": t_tr,
                        "gbs": round(step.transform_bytes() / (tr_ms * 1e-3) / 1e9, 1),
                        "hbm_frac": round(step.transform_bytes() / (tr_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                        "algorithmic_bytes": step.transform_bytes()}

    # the contraction on the ready window tensor
    step.transform()
    cbytes = step.contraction_bytes()
    if trace:
        cw = trace_stats(kernel_trace(step.stream, step.contract, iters))
        cc = trace_stats(kernel_trace(step.stream, step.contract, iters, flush))
        roof = roofline_entry(fl, cbytes, L.dtype, cw["dominant"], co_ms)
        roof["scope"] = "call: " + " + ".join(cw["kernels"]) + " (HIP events around back-to-back calls)"
        roof["kernel_only"] = roofline_entry(fl, cbytes, L.dtype, cw["dominant"], cw["dominant_us"]["median_us"] * 1e-3)
        roof["kernel_only"]["kernel"] = cw["dominant"]
        roof["kernel_only"]["scope"] = "dominant kernel's median traced duration (warm)"
    else:
        cw = cc = None
        roof = step.contraction_roofline(co_ms)
    roof["traffic"] = stored_traffic(traffic_key(L, epilogue))
    res["contraction"] = {"call_ms": round(co_ms, 5), "warm": cw, "cold": cc, "roofline": roof}

    # the in-LDS call (no window tensor in HBM)
    call, nbytes = implicit_call(step)
    if call is not None:
        settle(call)   # (the traces before ran cold passes: 1 GiB reads between calls)
    if call is not None and not trace:
        _, wall = loop_ms(step.stream, call, steps, warmup)
        ms, _ = call_ms(step.stream, call, steps, 1)
        res["in_lds"] = {"call_ms": round(ms, 5), "wall_ms": round(wall, 5), "workspace_bytes": nbytes,
                         "tflops": round(fl / (ms * 1e-3) / 1e12, 3)}
    elif call is not None:
        _, wall = loop_ms(step.stream, call, steps, warmup)
        ms, _ = call_ms(step.stream, call, steps, 1)
        iw = trace_stats(kernel_trace(step.stream, call, iters))
        ic = trace_stats(kernel_trace(step.stream, call, iters, flush))
        ibytes = step.bytes_x() + step.bytes_w() + step.bytes_b() + step.bytes_y()
        roof = roofline_entry(fl, ibytes, L.dtype, iw["dominant"], ms)
        roof["scope"] = "call: " + " + ".join(iw["kernels"]) + " (HIP events around back-to-back calls)"
        roof["kernel_only"] = roofline_entry(fl, ibytes, L.dtype, iw["dominant"], iw["dominant_us"]["median_us"] * 1e-3)
        roof["kernel_only"]["kernel"] = iw["dominant"]
        roof["kernel_only"]["scope"] = "dominant kernel's median traced duration (warm)"
        roof["kernel_only_cold"] = roofline_entry(fl, ibytes, L.dtype, iw["dominant"], ic["dominant_us"]["median_us"] * 1e-3)
        roof["traffic"] = stored_traffic(traffic_key(L, epilogue) + "+implicit")
        res["in_lds"] = {"call_ms": round(ms, 5), "wall_ms": round(wall, 5), "workspace_bytes": nbytes,
                         "tflops": round(fl / (ms * 1e-3) / 1e12, 3), "warm": iw, "cold": ic,
                         "roofline": roof}
    if epilogue != "none":
        res["epilogue"] = epilogue
        res["output_bytes"] = step.bytes_y()
        if unfused:
            # context: the plain contraction, then torch's ReLU (and pool)
            res["unfused_contract_ms"] = round(time_unfused(L, epilogue, steps, warmup), 5)
    return res, step


def cpu_oracle_point(L: workloads.Layer, seconds: float) -> dict:
    """The oracle (O1) on a bounded sample of the layer, as cpu_baseline."""
    return cpu_baseline(L, seconds)


def cpu_im2col_point(L: workloads.Layer, seconds: float) -> dict:
    """The numpy im2col + matmul convolution (O4, fp64) on whole images of the
    layer, as many as fit about `seconds`: the explicit-GEMM CPU point."""
    import oracle
    x, w, b = workloads.make_inputs(L)
    f = lambda a: None if a is None else workloads.to_f64(a, L.dtype)
    x, w, b = f(x), f(w), f(b)
    P, Q = oracle.out_dims(L.x_shape, L.w_shape, L.stride, L.pad, L.dil, L.groups)
    flops_img = 2 * L.K * (L.C // L.groups) * L.R * L.S * P * Q
    t0 = time.perf_counter()
    oracle.im2col_conv(x[:1], w, b, L.stride, L.pad, L.dil, L.groups)
    one = time.perf_counter() - t0
    want = max(1, int(seconds / max(one, 1e-6)))
    n_img = min(L.N, want)
    reps = max(1, want // n_img)
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.im2col_conv(x[:n_img], w, b, L.stride, L.pad, L.dil, L.groups)
    dt = time.perf_counter() - t0
    return {"value": round(flops_img * n_img * reps / dt / 1e12, 6), "unit": "TFLOP/s",
            "sample": f"{n_img} of {L.N} images x {reps} repeats ({dt:.2f} s wall); "
                      f"numpy fp64 im2col @ filter matrix"}


def ablation_report(runs: int = 5, calls: int = 50) -> dict:
    """The ablation variants (copies of the library with one kernel's
    optimizations switched off, built by cnn_convolution_im2win_amd.build)
    timed on the 128x64x56x56 fp16 layer through their C ABI: 10 warm-up
    calls, then `runs` runs of `calls` calls back to back, HIP events around
    each run; median, best and spread of the per-call means.  Parity of every
    variant is checked by tests/test_gpu_ablation.py, not here."""
    import torch
    from cnn_convolution_im2win_amd import _lib, build
    L = workloads.LAYERS["resnet_3x3_fp16"]
    x, w, _ = workloads.make_inputs(L)
    xd = torch.from_numpy(x).to("cuda")
    wd = torch.from_numpy(w).to("cuda")
    desc = _lib.ConvDesc(L.N, L.C, L.H, L.W, L.K, L.R, L.S, 1, 1, 1, 1, 1, 1, 1)
    y = torch.empty((L.N, L.K, L.H, L.W), dtype=torch.float16, device="cuda")
    stream = torch.cuda.Stream()
    out = {}
    for name, (_, _, what) in build.VARIANTS.items():
        lib = _lib.open_library(build.variant_path(name))
        nb = ctypes.c_size_t()
        implicit = name.startswith("implicit")
        flags = _lib.CIW_FLAG_IMPLICIT if implicit else 0
        if implicit:
            st = lib.conv2d_implicit_workspace_bytes(ctypes.byref(desc), 1, 1, flags, ctypes.byref(nb))
        else:
            st = lib.conv2d_workspace_bytes(ctypes.byref(desc), 1, L.N, ctypes.byref(nb))
        if st != 0:
            raise RuntimeError(f"{name}: workspace query status {st}")
        ws = torch.empty(max(nb.value, 16), dtype=torch.uint8, device="cuda")
        args = (ctypes.byref(desc), 1, 1, xd.data_ptr(), wd.data_ptr(), None, y.data_ptr(),
                ws.data_ptr(), nb.value, flags, stream.cuda_stream)

        def call():
            st = lib.conv2d_fwd(*args)
            if st != 0:
                raise RuntimeError(f"{name}: conv2d_fwd status {st}")
        for _ in range(10):
            call()
        torch.cuda.synchronize()
        ms = []
        for _ in range(runs):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(calls):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1) / calls)
        ms.sort()
        med = ms[len(ms) // 2]
        out[name] = {"what": what, "median_us": round(med * 1e3, 2), "best_us": round(ms[0] * 1e3, 2),
                     "worst_us": round(ms[-1] * 1e3, 2)}
        print(f"# ablation {name}: {json.dumps(out[name])}", file=sys.stderr, flush=True)
    for name, r in out.items():
        base = out[name.split("_", 1)[0] + "_baseline"]
        r["vs_baseline"] = round(r["median_us"] / base["median_us"], 3)
        # a difference counts only beyond both runs' spreads (worst - best)
        noise = (r["worst_us"] - r["best_us"]) + (base["worst_us"] - base["best_us"])
        r["beyond_noise"] = abs(r["median_us"] - base["median_us"]) > noise
    return {"layer": describe(L), "scope": "one conv2d_fwd call (materialised: repack + contraction "
            "+ filter re-layout; in-LDS: filter re-layout + contraction)", "runs": runs,
            "calls_per_run": calls, "variants": out}


def main():
    global SETTLE_S
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=workloads.LAYER_ORDER,
                    help="the layer the headline value is quoted on")
    ap.add_argument("--iters", type=int, default=50,
                    help="traced calls per regime (best and median are over these)")
    ap.add_argument("--headline-only", action="store_true",
                    help="measure only the headline layer (e.g. under a profiler)")
    ap.add_argument("--epilogue", default="none", choices=EPILOGUES,
                    help="fuse ReLU / ReLU + 2x2 max-pool into the contraction")
    ap.add_argument("--no-memory", action="store_true", help="skip the per-layer memory table")
    ap.add_argument("--no-trace", action="store_true",
                    help="skip the kernel traces (for runs under rocprofv3, which traces itself)")
    ap.add_argument("--no-unfused", action="store_true",
                    help="with --epilogue, skip the unfused comparison")
    ap.add_argument("--miopen", action="store_true",
                    help="add MIOpen's convolution (torch conv2d) to the memory table, as context")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time of the headline layer's oracle sample")
    ap.add_argument("--layer-cpu-seconds", type=float, default=3.0,
                    help="CPU time of each other layer's oracle sample and of the im2col point")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed back-to-back calls before each layer's timed loops "
                         "(0 under a profiler, whose records would grow with them)")
    ap.add_argument("--ablation", action="store_true",
                    help="time the ablation variant libraries instead (one JSON line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM counter scaling)")
    args = ap.parse_args()
    SETTLE_S = max(0.0, args.settle)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for {max(args.gpus, world)}): this "
              "library has no multi-GPU path; the per-GPU throughput at N=1 is the figure.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.ablation:
        print(json.dumps(ablation_report()), flush=True)
        return

    # reading 1 GiB evicts the L2 caches and the 256 MB Infinity Cache
    flush = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    names = [args.workload] if args.headline_only else \
        [args.workload] + [n for n in workloads.LAYER_ORDER if n != args.workload]
    layers, head_step = {}, None
    for name in names:
        L = workloads.LAYERS[name]
        print(f"# measuring {describe(L)} (epilogue {args.epilogue})", file=sys.stderr, flush=True)
        steps = args.steps if name == args.workload else max(10, args.steps // 5)
        warm = args.warmup if name == args.workload else min(args.warmup, 5)
        r, st = measure_layer2(L, steps, warm, args.iters, flush, args.epilogue,
                               trace=not args.no_trace, unfused=not args.no_unfused)
        k32 = time_fp32_kernels(st, steps, warm)
        if k32 is not None:
            r["fp32_kernels_forced"] = k32
        layers[name] = r
        if name == args.workload:
            head_step = st
        else:
            del st
        print(f"# {name}: {json.dumps(r)}", file=sys.stderr, flush=True)
    del flush

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        bb = torch.empty_like(a)
        for _ in range(3):
            bb.copy_(a)
        torch.cuda.synchronize()
        del a, bb

    if not args.no_memory and not args.headline_only:
        for name in names:
            print(f"# memory {name}", file=sys.stderr, flush=True)
            layers[name]["memory"] = memory_report(workloads.LAYERS[name], miopen=args.miopen,
                                                   epilogue=args.epilogue)

    cpu = None
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(workloads.LAYERS[args.workload], args.cpu_seconds)
        layers[args.workload]["cpu_oracle"] = cpu
        layers[args.workload]["cpu_im2col"] = cpu_im2col_point(workloads.LAYERS[args.workload],
                                                               args.layer_cpu_seconds)
        for name in names:
            if name == args.workload:
                continue
            layers[name]["cpu_oracle"] = cpu_oracle_point(workloads.LAYERS[name], args.layer_cpu_seconds)
        for name in names:
            r = layers[name]
            r["speedup_vs_oracle"] = {"step": round(r["step"]["tflops"] / r["cpu_oracle"]["value"], 1)}
            if "in_lds" in r:
                r["speedup_vs_oracle"]["in_lds"] = round(r["in_lds"]["tflops"] / r["cpu_oracle"]["value"], 1)

    head = layers[args.workload]
    L = workloads.LAYERS[args.workload]
    value = head_step.flops() / (head["step"]["ms"] * 1e-3) / 1e12
    page = PAGE_BASELINE.get(args.workload)
    roof = dict(head["contraction"]["roofline"])
    out = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": round(head["step"]["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        # the pages print one absolute time, for exactly this layer, on a
        # different machine (context, not a target); the same-box oracle
        # figure is cpu_baseline / vs_cpu_oracle
        "vs_baseline": round(value / page, 1) if page else None,
        "vs_baseline_basis": ("OpenCL-Benchmarks page: direct convolution of this layer on a "
                              "Mali T860, 913.301 ms (another machine; context only)") if page else None,
        "vs_cpu_oracle": round(value / cpu["value"], 1) if cpu else None,
        "dtype": L.dtype,
        "data": "synthetic",
        "config": {"workload": describe(L), "global_batch": L.N,
                   "step": "conv_im2win_transform + conv2d_fwd(window ready)",
                   "epilogue": "bias" + {"none": "", "relu": " + relu",
                                         "relu_pool": " + relu + 2x2 max-pool"}[args.epilogue],
                   "transform_ms": head["transform"]["call_ms"],
                   "contract_ms": head["contraction"]["call_ms"]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "layers": layers,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Bar: the window tensor is bit-exact (pitch tails included); outputs satisfy
max|y - ref| <= tol * max|ref| with tol = 1e-4 (fp32) and 2e-2 (fp16/bf16),
ref being the fp64 oracle on the same (exactly upcast) inputs.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import (TOL, host_bits, rel_err, sample_indices, to_dev, to_host_bits,
                            to_host_f64, torch_dtype)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import cnn_convolution_im2win_amd as ciw  # noqa: E402

CODE = {"f32": ciw.CIW_F32, "f16": ciw.CIW_F16, "bf16": ciw.CIW_BF16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def layer_inputs(L):
    x, w, b = workloads.make_inputs(L)
    return x, w, b


def run_gpu(L, x, w, b, flags=0, workspace_images=None, out_dtype=None):
    xd, wd, bd = to_dev(x, L.dtype), to_dev(w, L.dtype), to_dev(b, L.dtype)
    desc = ciw.make_desc(L.x_shape, L.w_shape, L.stride, L.pad, L.dil, L.groups)
    ws = None
    if workspace_images is not None:
        nbytes = ciw.conv2d_workspace_bytes(desc, CODE[L.dtype], workspace_images)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    od = torch_dtype(out_dtype or L.out_dtype)
    y = ciw.conv2d(xd, wd, bd, L.stride, L.pad, L.dil, L.groups, out_dtype=od, workspace=ws,
                   flags=flags)
    torch.cuda.synchronize()
    return y


def oracle_full(L, x, w, b):
    f = lambda a: None if a is None else workloads.to_f64(a, L.dtype)
    return oracle.conv2d(f(x), f(w), f(b), L.stride, L.pad, L.dil, L.groups)


def check_close(got, ref, dtype, what):
    e = rel_err(got, ref)
    say(f"  {what}: rel err {e:.3e} (tol {TOL[dtype]:.0e})")
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got))
    assert e <= TOL[dtype], what


# ------------------------------------------------------------------ repack
@pytest.mark.parametrize("name", workloads.LAYER_ORDER)
@pytest.mark.parametrize("layout", [0, 1])
def test_transform_bit_exact_full_layers(name, layout):
    L = workloads.LAYERS[name]
    say(f"transform {name} layout {layout} {L.x_shape}")
    x, _, _ = layer_inputs(L)
    xd = to_dev(x, L.dtype)
    got = ciw.conv_im2win_transform(xd, L.R, L.S, L.stride, L.pad, L.dil, layout)
    torch.cuda.synchronize()
    ref = oracle.im2win(x, L.R, L.S, L.stride, L.pad, L.dil, layout)
    assert tuple(got.shape) == ref.shape
    assert np.array_equal(to_host_bits(got), host_bits(ref))


def test_transform_bit_exact_random():
    rng = np.random.default_rng(2024)
    for i in range(40):
        dtype = ["f32", "f16", "bf16"][i % 3]
        L = workloads.random_layer(rng, dtype=dtype, max_hw=40, max_c=70)
        x, _, _ = layer_inputs(L)
        for layout in (0, 1):
            say(f"transform random #{i} {L.x_shape} R,S={L.R},{L.S} s={L.stride} p={L.pad} "
                f"d={L.dil} {dtype} layout {layout}")
            got = ciw.conv_im2win_transform(to_dev(x, dtype), L.R, L.S, L.stride, L.pad, L.dil,
                                            layout)
            torch.cuda.synchronize()
            ref = oracle.im2win(x, L.R, L.S, L.stride, L.pad, L.dil, layout)
            assert np.array_equal(to_host_bits(got), host_bits(ref))


def test_transform_wide_rows_column_tiled():
    # rows wider than the LDS tile: the column- and channel-tiled paths
    L = workloads.Layer("wide", N=1, C=5, H=6, W=3000, K=1, R=7, S=3, stride=(1, 2),
                        pad=(3, 1), dtype="f32")
    x, _, _ = layer_inputs(L)
    for layout in (0, 1):
        say(f"transform wide layout {layout}")
        got = ciw.conv_im2win_transform(to_dev(x, "f32"), L.R, L.S, L.stride, L.pad, L.dil,
                                        layout)
        torch.cuda.synchronize()
        ref = oracle.im2win(x, L.R, L.S, L.stride, L.pad, L.dil, layout)
        assert np.array_equal(to_host_bits(got), host_bits(ref))


# ------------------------------------------------------------------ full compare
@pytest.mark.parametrize("name", ["tiny_3x3_fp32", "mid_3x3_fp32"])
def test_fp32_layers_full(name):
    L = workloads.LAYERS[name]
    say(f"conv2d {name}")
    x, w, b = layer_inputs(L)
    ref = oracle_full(L, x, w, b)
    got = to_host_f64(run_gpu(L, x, w, b))
    check_close(got, ref, L.dtype, name)


@pytest.mark.parametrize("name,n", [("resnet_3x3_fp16", 2), ("stem_7x7_s2_bf16", 2),
                                    ("dw_3x3_fp32", 3)])
def test_big_layers_reduced_batch_full(name, n):
    # the full layer's shape with a small batch: every output compared
    L = workloads.LAYERS[name].replace(N=n)
    say(f"conv2d {name} N={n}")
    x, w, b = layer_inputs(L)
    ref = oracle_full(L, x, w, b)
    got = to_host_f64(run_gpu(L, x, w, b))
    check_close(got, ref, L.dtype, f"{name} N={n}")


@pytest.mark.parametrize("name", ["resnet_3x3_fp16", "stem_7x7_s2_bf16", "dw_3x3_fp32"])
def test_big_layers_full_size_sampled(name):
    # the full batch in the launch configuration the benchmark uses; outputs
    # checked at sampled points the oracle computes one by one
    L = workloads.LAYERS[name]
    say(f"conv2d {name} full size, sampled")
    x, w, b = layer_inputs(L)
    y = to_host_f64(run_gpu(L, x, w, b))
    rng = np.random.default_rng(77)
    idx = sample_indices(y.shape, 3000, rng)
    f = lambda a: None if a is None else workloads.to_f64(a, L.dtype)
    ref = oracle.conv2d_points(f(x), f(w), f(b), idx, L.stride, L.pad, L.dil, L.groups)
    got = y[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]]
    # scale: max |ref| over the sample (a lower bound of the full max)
    check_close(got, ref, L.dtype, f"{name} sampled")
    assert np.all(np.isfinite(y))


# ------------------------------------------------------------------ sweeps
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_random_dense_sweep(dtype):
    rng = np.random.default_rng({"f32": 1, "f16": 2, "bf16": 3}[dtype])
    for i in range(30):
        L = workloads.random_layer(rng, dtype=dtype, max_hw=20, max_c=40, max_k=80)
        say(f"dense #{i} {dtype} x{L.x_shape} w{L.w_shape} s={L.stride} p={L.pad} d={L.dil} "
            f"bias={L.b_dist is not None}")
        x, w, b = layer_inputs(L)
        ref = oracle_full(L, x, w, b)
        for flags in (0, ciw.CIW_FLAG_GENERIC):
            got = to_host_f64(run_gpu(L, x, w, b, flags=flags))
            check_close(got, ref, dtype, f"dense #{i} flags {flags}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_random_depthwise_sweep(dtype):
    rng = np.random.default_rng({"f32": 4, "f16": 5, "bf16": 6}[dtype])
    for i in range(20):
        L = workloads.random_layer(rng, dtype=dtype, depthwise=True, max_hw=24, max_c=40)
        say(f"depthwise #{i} {dtype} x{L.x_shape} R,S={L.R},{L.S} s={L.stride} p={L.pad} "
            f"d={L.dil}")
        x, w, b = layer_inputs(L)
        ref = oracle_full(L, x, w, b)
        for flags in (0, ciw.CIW_FLAG_GENERIC):
            got = to_host_f64(run_gpu(L, x, w, b, flags=flags))
            check_close(got, ref, dtype, f"depthwise #{i} flags {flags}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_half_inputs_fp32_output(dtype):
    L = workloads.LAYERS["resnet_3x3_fp16"].replace(N=1, dtype=dtype, out_dtype="f32",
                                                    b_dist=("uniform", -0.1, 0.1))
    say(f"{dtype} -> f32 output")
    x, w, b = layer_inputs(L)
    ref = oracle_full(L, x, w, b)
    got = to_host_f64(run_gpu(L, x, w, b, out_dtype="f32"))
    # fp32 output of half inputs: only fp32 accumulation error remains
    check_close(got, ref, "f32", f"{dtype}->f32")


# ------------------------------------------------------------------ chunking etc.
@pytest.mark.parametrize("name", ["mid_3x3_fp32", "resnet_3x3_fp16", "stem_7x7_s2_bf16",
                                  "dw_3x3_fp32"])
def test_chunked_equals_full_batch(name):
    L = workloads.LAYERS[name]
    L = L.replace(N=min(L.N, 5))
    say(f"chunking {name} N={L.N}")
    x, w, b = layer_inputs(L)
    full = to_host_bits(run_gpu(L, x, w, b))
    for imgs in (1, 2):
        part = to_host_bits(run_gpu(L, x, w, b, workspace_images=imgs))
        if L.dtype == "f32" and L.groups == 1:
            # the fp32 channel split depends on the chunk size; compare values
            got = to_host_f64(run_gpu(L, x, w, b, workspace_images=imgs))
            ref = oracle_full(L, x, w, b)
            check_close(got, ref, L.dtype, f"{name} chunk {imgs}")
        else:
            assert np.array_equal(part, full), f"{name} chunk {imgs}"


def test_fp32_split_and_no_split_agree():
    L = workloads.LAYERS["mid_3x3_fp32"]
    x, w, b = layer_inputs(L)
    ref = oracle_full(L, x, w, b)
    for flags in (0, ciw.CIW_FLAG_NO_SPLIT):
        say(f"mid fp32 flags {flags}")
        check_close(to_host_f64(run_gpu(L, x, w, b, flags=flags)), ref, "f32", f"flags {flags}")


@pytest.mark.parametrize("name", workloads.LAYER_ORDER)
def test_window_ready_path(name):
    # the contraction alone, on a window tensor made by conv_im2win_transform
    L = workloads.LAYERS[name]
    L = L.replace(N=min(L.N, 4))
    say(f"window-ready {name}")
    x, w, b = layer_inputs(L)
    xd, wd, bd = to_dev(x, L.dtype), to_dev(w, L.dtype), to_dev(b, L.dtype)
    desc = ciw.make_desc(L.x_shape, L.w_shape, L.stride, L.pad, L.dil, L.groups)
    layout = ciw.CIW_WIN_HWC if (L.dtype != "f32" and L.groups == 1) else ciw.CIW_WIN_CHW
    nbytes = ciw.conv2d_workspace_bytes(desc, CODE[L.dtype], L.N)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    rows, _, pitch = ciw.conv_im2win_window_geometry(desc, CODE[L.dtype], layout)
    xw = ws[: L.N * rows * pitch * xd.element_size()].view(xd.dtype).view(L.N * rows, pitch)
    ciw.conv_im2win_transform(xd, L.R, L.S, L.stride, L.pad, L.dil, layout, out=xw)
    P, Q = ciw.conv_im2win_output_dims(desc)
    y = torch.empty((L.N, L.K, P, Q), dtype=torch_dtype(L.out_dtype), device="cuda")
    fn = ciw.conv2d_dw_fwd if L.groups > 1 else ciw.conv2d_fwd
    fn(None, wd, bd, y, ws, L.stride, L.pad, L.dil, flags=ciw.CIW_FLAG_WINDOW_READY,
       x_shape=L.x_shape)
    torch.cuda.synchronize()
    ref = oracle_full(L, x, w, b)
    check_close(to_host_f64(y), ref, L.dtype, f"window-ready {name}")


def test_empty_batch():
    L = workloads.LAYERS["tiny_3x3_fp32"]
    xd = torch.empty((0, 16, 32, 32), device="cuda")
    wd = to_dev(workloads.make_inputs(L)[1], "f32")
    y = ciw.conv2d(xd, wd, None, 1, 1)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, 32, 32, 32)


def test_errors_raise():
    L = workloads.LAYERS["tiny_3x3_fp32"]
    x, w, b = layer_inputs(L)
    xd, wd = to_dev(x, "f32"), to_dev(w, "f32")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ciw.Im2winError):
        ciw.conv2d(xd, wd, None, 1, 1, workspace=ws)
    with pytest.raises(ValueError):
        ciw.conv2d(xd, wd[:, :8].contiguous(), None, 1, 1)

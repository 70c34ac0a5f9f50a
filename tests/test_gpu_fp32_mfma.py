"""GPU parity of the fp32 matrix-core contraction (forced with
CIW_FLAG_FP32_MFMA: 3x3 and 1x1 fp32 layers with output rows of at most 192
pixels take it; CIW_FLAG_NO_SPLIT and the 2x2 pool keep the vector-ALU
kernel), and of the automatic choice on the mid layer.  Bar: max|y - ref| <= 1e-4 * max|ref|
against the fp64 oracle, every output."""
import sys

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import TOL, rel_err, to_dev, to_host_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import cnn_convolution_im2win_amd as ciw  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# (N, C, H, W, K, R, stride, pad, dil): channel slices of 4..32 with a
# ragged last one, odd C, K not a multiple of 64, several pixel blocks per
# image, strides, dilation, 1x1, rows of exactly 192 pixels
SHAPES = [
    (1, 512, 13, 13, 1024, 3, 1, 1, 1),
    (1, 16, 32, 32, 32, 3, 1, 1, 1),
    (2, 37, 11, 9, 70, 3, 1, 1, 1),
    (1, 64, 30, 30, 65, 3, 2, 1, 1),
    (3, 24, 15, 17, 40, 3, 1, 2, 2),
    (1, 130, 7, 7, 200, 1, 1, 0, 1),
    (2, 5, 9, 192, 9, 1, 1, 0, 1),
    (1, 3, 20, 14, 64, 3, 1, 0, 1),
    (4, 96, 14, 14, 128, 3, 1, 1, 1),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("relu", [False, True])
def test_fp32_mfma_against_oracle(shape, relu):
    N, C, H, W, K, R, s, p, d = shape
    L = workloads.Layer("f32m", N=N, C=C, H=H, W=W, K=K, R=R, S=R, stride=(s, s), pad=(p, p),
                        dil=(d, d), x_dist=("uniform", -1.0, 1.0), seed=sum(shape) + relu)
    say(f"fp32 mfma {shape} relu={relu}")
    x, w, b = workloads.make_inputs(L)
    flags = ciw.CIW_FLAG_FP32_MFMA | (ciw.CIW_FLAG_RELU if relu else 0)
    y = ciw.conv2d(to_dev(x, "f32"), to_dev(w, "f32"), to_dev(b, "f32"), L.stride, L.pad, L.dil,
                   flags=flags)
    torch.cuda.synchronize()
    got = to_host_f64(y)
    ref = oracle.conv2d(x.astype(np.float64), w.astype(np.float64), b.astype(np.float64),
                        L.stride, L.pad, L.dil, 1)
    if relu:
        ref = oracle.relu_pool(ref, relu=True, pool=False)
    e = rel_err(got, ref)
    say(f"  rel err {e:.3e}")
    assert got.shape == ref.shape and np.all(np.isfinite(got))
    assert e <= TOL["f32"]


@pytest.mark.parametrize("flags", ["default", "valu", "mfma"])
def test_mid_layer_each_kernel_choice(flags):
    """The 1x512x13x13 -> 1024 layer through the automatic choice and each
    forced kernel (the vector kernel with its split channel sum)."""
    L = workloads.LAYERS["mid_3x3_fp32"]
    x, w, b = workloads.make_inputs(L)
    fl = {"default": 0, "valu": ciw.CIW_FLAG_FP32_VALU, "mfma": ciw.CIW_FLAG_FP32_MFMA}[flags]
    y = ciw.conv2d(to_dev(x, "f32"), to_dev(w, "f32"), to_dev(b, "f32"), 1, 1, flags=fl)
    torch.cuda.synchronize()
    ref = oracle.conv2d(x.astype(np.float64), w.astype(np.float64), b.astype(np.float64), 1, 1, 1, 1)
    e = rel_err(to_host_f64(y), ref)
    say(f"mid layer {flags}: rel err {e:.3e}")
    assert e <= TOL["f32"]


def test_fp32_mfma_pool_keeps_vector_kernel():
    L = workloads.LAYERS["mid_3x3_fp32"]
    x, w, b = workloads.make_inputs(L)
    fl = ciw.CIW_FLAG_FP32_MFMA | ciw.CIW_FLAG_RELU | ciw.CIW_FLAG_MAXPOOL2
    y = ciw.conv2d(to_dev(x, "f32"), to_dev(w, "f32"), to_dev(b, "f32"), 1, 1, flags=fl)
    torch.cuda.synchronize()
    ref = oracle.relu_pool(oracle.conv2d(x.astype(np.float64), w.astype(np.float64),
                                         b.astype(np.float64), 1, 1, 1, 1), relu=True, pool=True)
    assert rel_err(to_host_f64(y), ref) <= TOL["f32"]


def test_fp32_mfma_deterministic():
    L = workloads.LAYERS["mid_3x3_fp32"]
    x, w, b = workloads.make_inputs(L)
    xd, wd, bd = to_dev(x, "f32"), to_dev(w, "f32"), to_dev(b, "f32")
    y0 = ciw.conv2d(xd, wd, bd, 1, 1, flags=ciw.CIW_FLAG_FP32_MFMA)
    y1 = ciw.conv2d(xd, wd, bd, 1, 1, flags=ciw.CIW_FLAG_FP32_MFMA)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


@pytest.mark.parametrize("imgs", [1, 3])
def test_fp32_mfma_batch_chunks(imgs):
    """A 4-image fp32 layer whose plan takes the matrix cores, run in chunks
    of 1 or 3 images through one workspace (the partial sums of every chunk
    in the same buffer), against the oracle."""
    L = workloads.Layer("f32chunk", N=4, C=96, H=14, W=14, K=128, R=3, S=3, stride=(1, 1),
                        pad=(1, 1), x_dist=("uniform", -1.0, 1.0), seed=11)
    x, w, b = workloads.make_inputs(L)
    desc = ciw.make_desc(L.x_shape, L.w_shape, L.stride, L.pad, L.dil, 1)
    ws = torch.empty(ciw.conv2d_workspace_bytes(desc, ciw.CIW_F32, imgs), dtype=torch.uint8,
                     device="cuda")
    y = ciw.conv2d(to_dev(x, "f32"), to_dev(w, "f32"), to_dev(b, "f32"), 1, 1, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.conv2d(x.astype(np.float64), w.astype(np.float64), b.astype(np.float64), 1, 1, 1, 1)
    e = rel_err(to_host_f64(y), ref)
    say(f"fp32 chunks of {imgs}: rel err {e:.3e}")
    assert e <= TOL["f32"]


@pytest.mark.parametrize("forced", [ciw.CIW_FLAG_FP32_MFMA, ciw.CIW_FLAG_FP32_VALU])
def test_fp32_uneven_chunks_odd_plane(forced):
    """K * P * Q odd and a workspace for 5 of 9 images: the second chunk's
    output starts at a byte offset that is not a multiple of 16 (4 images x
    3 x 13 x 13 floats), which the slice reduction must handle (no 16-byte
    stores to it)."""
    L = workloads.Layer("f32odd", N=9, C=64, H=13, W=13, K=3, R=3, S=3, stride=(1, 1),
                        pad=(1, 1), x_dist=("uniform", -1.0, 1.0), seed=23)
    x, w, b = workloads.make_inputs(L)
    desc = ciw.make_desc(L.x_shape, L.w_shape, L.stride, L.pad, L.dil, 1)
    ws = torch.empty(ciw.conv2d_workspace_bytes(desc, ciw.CIW_F32, 5), dtype=torch.uint8,
                     device="cuda")
    y = ciw.conv2d(to_dev(x, "f32"), to_dev(w, "f32"), to_dev(b, "f32"), 1, 1, workspace=ws,
                   flags=forced)
    torch.cuda.synchronize()
    ref = oracle.conv2d(x.astype(np.float64), w.astype(np.float64), b.astype(np.float64), 1, 1, 1, 1)
    e = rel_err(to_host_f64(y), ref)
    say(f"fp32 odd plane, chunks of 5 ({forced:#x}): rel err {e:.3e}")
    assert e <= TOL["f32"]

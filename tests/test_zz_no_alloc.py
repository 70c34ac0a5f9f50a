"""GPU check of conv2d_fwd_noalloc, the entry point that takes no workspace
and allocates nothing (its workspace is the library's own device array).

Each case makes two calls in a row through the C ABI, the second on a
smaller input, and compares each call's output with conv2d_fwd's on the
same input (given a workspace of its own), to the bar of the method:
max|y - y_ref| <= tol * max|y_ref| (1e-4 fp32, 2e-2 fp16).  The batch
chunking of the two calls may differ (the array holds a limited number of
images), which can only reorder fp32 partial sums; the fp16 row kernel's
sums do not depend on the chunk, so there the outputs must be bit-equal.
The smaller call is also checked against the fp64 oracle."""
import ctypes
import sys

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import TOL, rel_err, to_dev, to_host_bits, to_host_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import cnn_convolution_im2win_amd as ciw  # noqa: E402
from cnn_convolution_im2win_amd import _lib  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CODE = {"f32": _lib.CIW_F32, "f16": _lib.CIW_F16, "bf16": _lib.CIW_BF16}


def run_both(L, flags):
    """(noalloc output, conv2d_fwd output) for layer L, both through the C ABI."""
    x, w, b = workloads.make_inputs(L)
    xd, wd, bd = to_dev(x, L.dtype), to_dev(w, L.dtype), to_dev(b, L.dtype)
    desc = ciw.make_desc(L.x_shape, L.w_shape, L.stride, L.pad, L.dil, 1)
    P, Q = ciw.conv2d_output_dims(desc, flags)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[L.out_dtype]
    y_na = torch.full((L.N, L.K, P, Q), float("nan"), dtype=tdt, device="cuda")
    y_ref = torch.full_like(y_na, float("nan"))
    lib = _lib.load()
    stream = torch.cuda.current_stream().cuda_stream
    bptr = None if bd is None else bd.data_ptr()
    st = lib.conv2d_fwd_noalloc(ctypes.byref(desc), CODE[L.dtype], CODE[L.out_dtype], xd.data_ptr(),
                                wd.data_ptr(), bptr, y_na.data_ptr(), flags, stream)
    assert st == _lib.CIW_OK, _lib.status_string(st)
    if flags & _lib.CIW_FLAG_IMPLICIT:
        nbytes = ciw.conv2d_implicit_workspace_bytes(desc, CODE[L.dtype], CODE[L.out_dtype], flags)
    else:
        nbytes = ciw.conv2d_workspace_bytes(desc, CODE[L.dtype], L.N)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    st = lib.conv2d_fwd(ctypes.byref(desc), CODE[L.dtype], CODE[L.out_dtype], xd.data_ptr(),
                        wd.data_ptr(), bptr, y_ref.data_ptr(), ws.data_ptr(), nbytes, flags, stream)
    assert st == _lib.CIW_OK, _lib.status_string(st)
    torch.cuda.synchronize()
    return (x, w, b), y_na, y_ref


RESNET = workloads.LAYERS["resnet_3x3_fp16"]
MID = workloads.LAYERS["mid_3x3_fp32"]

# (first layer, second smaller layer, flags): the fp16 layer with 40 images
# needs two chunks of the 32 MiB array (one image's window tensor is 1.25 MB)
CASES = {
    "fp16_chunked": (RESNET.replace(N=40), RESNET.replace(N=3), 0),
    "fp16_in_lds": (RESNET.replace(N=8), RESNET.replace(N=2), _lib.CIW_FLAG_IMPLICIT),
    "fp32_mid": (MID, MID.replace(C=64, K=128, seed=9), 0),
    "fp16_relu_pool": (RESNET.replace(N=30), RESNET.replace(N=1, H=20, W=24),
                       _lib.CIW_FLAG_RELU | _lib.CIW_FLAG_MAXPOOL2),
}


@pytest.mark.parametrize("case", list(CASES))
def test_noalloc_two_calls_match_conv2d_fwd(case):
    first, second, flags = CASES[case]
    for i, L in enumerate((first, second)):
        say(f"noalloc {case} call {i + 1}: N={L.N} C={L.C} H={L.H} W={L.W} K={L.K} {L.dtype}")
        (x, w, b), y_na, y_ref = run_both(L, flags)
        got, ref = to_host_f64(y_na), to_host_f64(y_ref)
        assert np.all(np.isfinite(got))
        e = rel_err(got, ref)
        same = np.array_equal(to_host_bits(y_na), to_host_bits(y_ref))
        say(f"  against conv2d_fwd: rel err {e:.3e}, bit-equal {same}")
        assert e <= TOL[L.dtype]
        if L.dtype == "f16":
            assert same
        if i == 1:
            f64 = lambda a: None if a is None else workloads.to_f64(a, L.dtype)
            o = oracle.conv2d(f64(x), f64(w), f64(b), L.stride, L.pad, L.dil, 1)
            o = oracle.relu_pool(o, relu=bool(flags & _lib.CIW_FLAG_RELU),
                                 pool=bool(flags & _lib.CIW_FLAG_MAXPOOL2))
            eo = rel_err(got, o)
            say(f"  against the oracle: rel err {eo:.3e}")
            assert eo <= TOL[L.dtype]

"""GPU parity of the ablation variants: copies of the library in which one
kernel is built with some of its optimizations switched off (the im2win
paper, "Enabling Memory-efficient Im2win Convolution ...", §IV-E, ablates
its tensor-core kernel the same way).  Each variant must

  * match the fp64 oracle (O1) on the 128x64x56x56 fp16 layer: every output
    at a batch of 2, and 1000 sampled outputs at the full batch of 128 (the
    launch configuration the benchmark times), within 2e-2 * max|ref|;
  * equal the baseline build of the same kernel bit for bit: the switches
    change when and how data moves (copy-ahead depth, copy path, workgroup
    placement, LDS padding, where indices are computed), never the order of
    the sums, so any difference is a race or a lost copy.

The variant libraries are built by ``cnn_convolution_im2win_amd.build``
(``build_variants``, called from ``__graft_entry__.build()``)."""
import ctypes
import sys

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import TOL, rel_err, sample_indices, to_dev, to_host_bits, to_host_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from cnn_convolution_im2win_amd import _lib, build  # noqa: E402

RESNET = workloads.LAYERS["resnet_3x3_fp16"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


_libs = {}


def variant_lib(name):
    if name not in _libs:
        _libs[name] = _lib.open_library(build.variant_path(name))
    return _libs[name]


def kernel_of(name):
    return name.split("_", 1)[0]      # "rows" or "implicit"


def run_variant(name, L, x, w):
    """conv2d_fwd through the variant's C ABI: the materialised path (repack
    + row kernel) for "rows_*", CIW_FLAG_IMPLICIT for "implicit_*"."""
    lib = variant_lib(name)
    xd, wd = to_dev(x, "f16"), to_dev(w, "f16")
    desc = _lib.ConvDesc(L.N, L.C, L.H, L.W, L.K, L.R, L.S, L.stride[0], L.stride[1], L.pad[0],
                         L.pad[1], L.dil[0], L.dil[1], 1)
    P, Q = oracle.out_dims(L.x_shape, L.w_shape, L.stride, L.pad, L.dil, 1)
    y = torch.empty((L.N, L.K, P, Q), dtype=torch.float16, device="cuda")
    nbytes = ctypes.c_size_t()
    if kernel_of(name) == "implicit":
        flags = _lib.CIW_FLAG_IMPLICIT
        st = lib.conv2d_implicit_workspace_bytes(ctypes.byref(desc), _lib.CIW_F16, _lib.CIW_F16, flags,
                                                 ctypes.byref(nbytes))
    else:
        flags = 0
        st = lib.conv2d_workspace_bytes(ctypes.byref(desc), _lib.CIW_F16, L.N, ctypes.byref(nbytes))
    assert st == _lib.CIW_OK, st
    ws = torch.empty(max(nbytes.value, 16), dtype=torch.uint8, device="cuda")
    st = lib.conv2d_fwd(ctypes.byref(desc), _lib.CIW_F16, _lib.CIW_F16, xd.data_ptr(), wd.data_ptr(),
                        None, y.data_ptr(), ws.data_ptr(), nbytes.value, flags,
                        torch.cuda.current_stream().cuda_stream)
    assert st == _lib.CIW_OK, st
    torch.cuda.synchronize()
    return y


def f64(a):
    return workloads.to_f64(a, "f16")


@pytest.mark.parametrize("name", list(build.VARIANTS))
def test_variant_against_oracle_small_batch(name):
    L = RESNET.replace(N=2)
    say(f"ablation {name}: N=2, every output")
    x, w, _ = workloads.make_inputs(L)
    got = to_host_f64(run_variant(name, L, x, w))
    ref = oracle.conv2d(f64(x), f64(w), None, L.stride, L.pad, L.dil, 1)
    e = rel_err(got, ref)
    say(f"  rel err {e:.3e}")
    assert got.shape == ref.shape and e <= TOL["f16"]


@pytest.mark.parametrize("name", list(build.VARIANTS))
def test_variant_full_batch_sampled_and_bit_equal_to_baseline(name):
    L = RESNET
    say(f"ablation {name}: full batch")
    x, w, _ = workloads.make_inputs(L)
    y = run_variant(name, L, x, w)
    got = to_host_f64(y)
    idx = sample_indices(got.shape, 1000, np.random.default_rng(17))
    ref = oracle.conv2d_points(f64(x), f64(w), None, idx, L.stride, L.pad, L.dil, 1)
    e = rel_err(got[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]], ref)
    say(f"  sampled rel err {e:.3e}")
    assert e <= TOL["f16"]
    base = kernel_of(name) + "_baseline"
    if name != base:
        yb = run_variant(base, L, x, w)
        same = np.array_equal(to_host_bits(y), to_host_bits(yb))
        say(f"  bit-equal to {base}: {same}")
        assert same

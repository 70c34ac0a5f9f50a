"""GPU parity of the fp16/bf16 row kernel across its layouts, against the oracle.

The persistent MFMA row kernel specialises on the geometry of a layer: the
pad-chunk period of its LDS row layout (1, 2, 4, 8), the number of pixel
phases (1, 2, 4, 8) and filter sets, whether reduction steps need edge
masks, whether output rows are whole 16-byte vectors, and the ring depth.
Each layer below was chosen to land on one of those combinations (noted
beside it); every output is compared with the fp64 oracle.  The last test
puts one infinity into the input: only outputs whose window holds it may be
non-finite, which checks that window entries outside a pixel's window never
reach its sum.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from tests import row_kernel_cases
from tests.gpu_util import TOL, rel_err, to_dev, to_host_f64, torch_dtype

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import cnn_convolution_im2win_amd as ciw  # noqa: E402

CASES = row_kernel_cases.CASES


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run(Lr, x, w, b):
    y = ciw.conv2d(to_dev(x, Lr.dtype), to_dev(w, Lr.dtype), to_dev(b, Lr.dtype), Lr.stride,
                   Lr.pad, Lr.dil, Lr.groups, out_dtype=torch_dtype(Lr.out_dtype))
    torch.cuda.synchronize()
    return to_host_f64(y)


def reference(Lr, x, w, b):
    f = lambda a: None if a is None else workloads.to_f64(a, Lr.dtype)
    return oracle.conv2d(f(x), f(w), f(b), Lr.stride, Lr.pad, Lr.dil, Lr.groups)


@pytest.mark.parametrize("name", list(CASES))
def test_row_kernel_layouts(name):
    Lr = CASES[name]
    say(f"row kernel {name}: x{Lr.x_shape} w{Lr.w_shape} s={Lr.stride} p={Lr.pad} "
        f"{Lr.dtype}->{Lr.out_dtype}")
    x, w, b = workloads.make_inputs(Lr)
    ref = reference(Lr, x, w, b)
    got = run(Lr, x, w, b)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got))
    tol = TOL["f32"] if Lr.out_dtype == "f32" else TOL[Lr.dtype]
    # fp32 output of half inputs keeps only the fp32 accumulation error
    assert rel_err(got, ref) <= tol, name


@pytest.mark.parametrize("name", ["pad8_c64_k40", "stem_small", "pad1_c40"])
def test_row_kernel_infinity_stays_in_its_windows(name):
    Lr = CASES[name]
    say(f"row kernel {name} with one infinite input")
    x, w, b = workloads.make_inputs(Lr)
    x = x.copy()
    n, c, h, wi = 0, Lr.C // 2, Lr.H // 2, Lr.W // 2
    x[n, c, h, wi] = workloads.from_f64(np.array([np.inf]), Lr.dtype)[0]
    ref = reference(Lr, x, w, b)
    got = run(Lr, x, w, b)
    bad_ref = ~np.isfinite(ref)
    assert bad_ref.any()
    # exactly the outputs whose window holds the infinity are non-finite
    assert np.array_equal(~np.isfinite(got), bad_ref)
    tol = TOL["f32"] if Lr.out_dtype == "f32" else TOL[Lr.dtype]
    assert rel_err(got[~bad_ref], ref[~bad_ref]) <= tol

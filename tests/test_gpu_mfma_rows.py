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
from tests.gpu_util import TOL, rel_err, to_dev, to_host_f64, torch_dtype

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import cnn_convolution_im2win_amd as ciw  # noqa: E402

L = workloads.Layer
CASES = {
    # pad 8 (G = 24), no masks, K = 40: the second channel half partly valid
    "pad8_c64_k40": L("c", N=2, C=64, H=7, W=29, K=40, R=3, S=3, pad=(1, 1), dtype="f16",
                      out_dtype="f16"),
    # stride 2: pad 8, masked tail
    "pad8_c32_s2": L("c", N=2, C=32, H=9, W=37, K=64, R=3, S=3, stride=(2, 2), pad=(1, 1),
                     dtype="bf16", out_dtype="bf16"),
    # pad 4 (G = 12), two pixel blocks, fp32 output
    "pad4_c32_f32out": L("c", N=1, C=32, H=6, W=45, K=24, R=3, S=3, pad=(1, 1), dtype="f16",
                         out_dtype="f32"),
    # pad 2 (G = 6), Q = 13: element stores
    "pad2_c16_q13": L("c", N=3, C=16, H=5, W=13, K=64, R=3, S=3, pad=(1, 1), dtype="f16",
                      out_dtype="f16"),
    # G = 15 odd: no pad chunks, masked
    "pad1_c40": L("c", N=1, C=40, H=5, W=33, K=50, R=3, S=3, pad=(1, 1), dtype="bf16",
                  out_dtype="bf16"),
    # 1x1, G = 16: pad period capped at 8, vector stores
    "pad8cap_1x1_c128": L("c", N=2, C=128, H=4, W=40, K=64, R=1, S=1, dtype="f16",
                          out_dtype="f16"),
    # 1x1, G = 1, three pixel blocks, fp32 output
    "pad1_1x1_c8": L("c", N=2, C=8, H=5, W=70, K=17, R=1, S=1, dtype="bf16", out_dtype="f32"),
    # D = 18: four phases, two filter sets, shortened ring
    "nset2_c6": L("c", N=2, C=6, H=7, W=50, K=64, R=3, S=3, pad=(1, 1), dtype="f16",
                  out_dtype="f16"),
    # D = 9: eight phases, four filter sets
    "nset4_c3": L("c", N=2, C=3, H=6, W=90, K=33, R=3, S=3, pad=(1, 1), dtype="bf16",
                  out_dtype="bf16"),
    # D = 36: two phases, one set
    "nph2_c12": L("c", N=1, C=12, H=6, W=41, K=64, R=3, S=3, pad=(1, 1), dtype="f16",
                  out_dtype="f16"),
    # the 7x7 stride-2 stem on a smaller image
    "stem_small": L("c", N=1, C=3, H=30, W=75, K=64, R=7, S=7, stride=(2, 2), pad=(3, 3),
                    dtype="bf16", out_dtype="bf16"),
    # K = 20: the second channel half has no valid channel
    "k20_c64": L("c", N=1, C=64, H=5, W=17, K=20, R=3, S=3, pad=(1, 1), dtype="f16",
                 out_dtype="f16"),
    # a row needing all eight copy instructions per thread
    "long_row_c64": L("c", N=1, C=64, H=3, W=70, K=64, R=3, S=3, pad=(1, 1), dtype="f16",
                      out_dtype="f16"),
    # 1x5 filter, G = 6: pad 2
    "c48_1x5": L("c", N=2, C=48, H=9, W=21, K=64, R=1, S=5, pad=(0, 2), dtype="bf16",
                 out_dtype="bf16"),
}


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

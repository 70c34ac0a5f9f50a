"""GPU parity of the in-LDS window paths (CIW_FLAG_IMPLICIT): conv2d_fwd for
fp16/bf16 and conv2d_dw_fwd for every input type.

The kernels build their windows in LDS from x and never write the window
tensor; they must meet the same bar as the materialised path against the
fp64 oracle: max|y - ref| <= tol * max|ref|, tol 1e-4 for fp32 and 2e-2 for
fp16/bf16 inputs.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import TOL, rel_err, sample_indices, to_dev, to_host_f64, torch_dtype

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import cnn_convolution_im2win_amd as ciw  # noqa: E402

CODE = {"f32": ciw.CIW_F32, "f16": ciw.CIW_F16, "bf16": ciw.CIW_BF16}
IMP = ciw.CIW_FLAG_IMPLICIT


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(a, dt):
    return None if a is None else workloads.to_f64(a, dt)


def run(L, x, w, b, flags=IMP, out_dtype=None):
    xd, wd, bd = to_dev(x, L.dtype), to_dev(w, L.dtype), to_dev(b, L.dtype)
    od = torch_dtype(out_dtype or L.out_dtype)
    y = ciw.conv2d(xd, wd, bd, L.stride, L.pad, L.dil, 1, out_dtype=od, flags=flags)
    torch.cuda.synchronize()
    return y


def check(got, ref, what):
    e = rel_err(got, ref)
    say(f"  {what}: rel err {e:.3e}")
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got))
    assert e <= TOL["f16"], what


RESNET = workloads.LAYERS["resnet_3x3_fp16"]


@pytest.mark.parametrize("n", [1, 3])
def test_resnet_layer_reduced_batch_full(n):
    L = RESNET.replace(N=n)
    say(f"implicit resnet_3x3_fp16 N={n}, every output")
    x, w, b = workloads.make_inputs(L)
    got = to_host_f64(run(L, x, w, b))
    ref = oracle.conv2d(f64(x, "f16"), f64(w, "f16"), None, L.stride, L.pad, L.dil, 1)
    check(got, ref, f"N={n}")


def test_resnet_layer_full_size_sampled():
    """The full batch in the launch configuration the benchmark times;
    outputs checked at sampled points the oracle computes one by one, and
    every output against the materialised path."""
    L = RESNET
    say("implicit resnet_3x3_fp16 full size, sampled")
    x, w, b = workloads.make_inputs(L)
    y = run(L, x, w, b)
    got_all = to_host_f64(y)
    rng = np.random.default_rng(91)
    idx = sample_indices(got_all.shape, 3000, rng)
    ref = oracle.conv2d_points(f64(x, "f16"), f64(w, "f16"), None, idx, L.stride, L.pad, L.dil, 1)
    check(got_all[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]], ref, "sampled")
    explicit = to_host_f64(run(L, x, w, b, flags=0))
    check(got_all, explicit, "against the materialised path")


# (N, C, H, W, K, R, stride_w, pad, dil) -- every combination of compiled
# filter shape, channel-half count, partial pixel blocks, padding, stride and
# dilation the kernel distinguishes
SHAPES = [
    (2, 16, 9, 16, 8, 3, 1, 1, 1),
    (1, 32, 7, 24, 40, 3, 1, 1, 1),
    (2, 48, 6, 8, 33, 3, 2, 2, 1),
    (1, 64, 5, 40, 64, 3, 1, 1, 1),
    (3, 64, 12, 32, 17, 3, 1, 1, 1),
    (1, 16, 11, 16, 24, 3, 1, 2, 2),
    (2, 32, 4, 8, 64, 1, 1, 0, 1),
    (1, 64, 6, 72, 24, 1, 2, 1, 1),
    (1, 16, 3, 8, 1, 1, 1, 0, 1),
    (1, 64, 2, 8, 64, 3, 1, 1, 1),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype,out", [("f16", "f16"), ("bf16", "bf16"), ("f16", "f32"),
                                       ("bf16", "f32")])
def test_shapes_against_oracle(shape, dtype, out):
    N, C, H, W, K, R, sw, pad, dil = shape
    L = workloads.Layer("imp", N=N, C=C, H=H, W=W, K=K, R=R, S=R, stride=(1, sw),
                        pad=(pad, pad), dil=(dil, dil), dtype=dtype, out_dtype=out,
                        x_dist=("normal", 0.0, 1.0), seed=sum(shape))
    say(f"implicit {shape} {dtype}->{out}")
    x, w, b = workloads.make_inputs(L)
    got = to_host_f64(run(L, x, w, b))
    ref = oracle.conv2d(f64(x, dtype), f64(w, dtype), f64(b, dtype), L.stride, L.pad, L.dil, 1)
    check(got, ref, f"{shape} {dtype}->{out}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_relu_and_no_bias(dtype):
    L = workloads.Layer("imp", N=2, C=64, H=10, W=16, K=48, R=3, S=3, stride=(1, 1),
                        pad=(1, 1), dtype=dtype, out_dtype=dtype, x_dist=("normal", 0.0, 1.0),
                        b_dist=None, seed=5)
    x, w, _ = workloads.make_inputs(L)
    got = to_host_f64(run(L, x, w, None, flags=IMP | ciw.CIW_FLAG_RELU))
    ref = oracle.relu_pool(oracle.conv2d(f64(x, dtype), f64(w, dtype), None, L.stride, L.pad,
                                         L.dil, 1), relu=True, pool=False)
    check(got, ref, f"relu {dtype}")
    assert np.all(got >= 0)


# the fused epilogue: 2x2 max-pool (stride 2, floor), with or without ReLU
POOL_SHAPES = [s for s in SHAPES if s[2] >= 2] + [
    (2, 32, 9, 16, 40, 3, 1, 1, 1),     # P = 9: the last output row has no pair
    (1, 64, 7, 56, 64, 3, 1, 1, 1),     # pooled rows of 28: 4-element stores
    (1, 16, 6, 40, 8, 1, 2, 0, 1),      # Q = 20, pooled 10: 2-element stores
]


@pytest.mark.parametrize("shape", POOL_SHAPES)
@pytest.mark.parametrize("dtype,out,relu", [("f16", "f16", True), ("bf16", "bf16", False),
                                            ("f16", "f32", False), ("bf16", "f32", True)])
def test_pool_shapes_against_oracle(shape, dtype, out, relu):
    N, C, H, W, K, R, sw, pad, dil = shape
    L = workloads.Layer("imp", N=N, C=C, H=H, W=W, K=K, R=R, S=R, stride=(1, sw),
                        pad=(pad, pad), dil=(dil, dil), dtype=dtype, out_dtype=out,
                        x_dist=("normal", 0.0, 1.0), seed=sum(shape) + 3)
    P, Q = oracle.out_dims(L.x_shape, L.w_shape, L.stride, L.pad, L.dil, 1)
    if P < 2 or Q < 2:
        pytest.skip("no 2x2 region")
    say(f"implicit pool {shape} {dtype}->{out} relu={relu}")
    x, w, b = workloads.make_inputs(L)
    flags = IMP | ciw.CIW_FLAG_MAXPOOL2 | (ciw.CIW_FLAG_RELU if relu else 0)
    got = to_host_f64(run(L, x, w, b, flags=flags))
    conv = oracle.conv2d(f64(x, dtype), f64(w, dtype), f64(b, dtype), L.stride, L.pad, L.dil, 1)
    ref = oracle.relu_pool(conv, relu=relu, pool=True)
    check(got, ref, f"pool {shape} {dtype}->{out} relu={relu}")


def test_resnet_layer_relu_pool_full_size():
    """The full batch with ReLU and the 2x2 pool fused, in the launch
    configuration the benchmark times: every output against the
    materialised path's fused epilogue, and sampled outputs against the
    oracle (each the maximum of its four convolution outputs)."""
    L = RESNET
    say("implicit resnet_3x3_fp16 full size, relu + pool")
    x, w, b = workloads.make_inputs(L)
    flags = ciw.CIW_FLAG_RELU | ciw.CIW_FLAG_MAXPOOL2
    got_all = to_host_f64(run(L, x, w, b, flags=IMP | flags))
    assert got_all.shape == (L.N, L.K, 28, 28)
    explicit = to_host_f64(run(L, x, w, b, flags=flags))
    check(got_all, explicit, "against the materialised path")
    rng = np.random.default_rng(92)
    idx = sample_indices(got_all.shape, 1000, rng)
    quad = np.concatenate([idx * [1, 1, 2, 2] + [0, 0, dy, dx] for dy in (0, 1) for dx in (0, 1)])
    pts = oracle.conv2d_points(f64(x, "f16"), f64(w, "f16"), None, quad, L.stride, L.pad, L.dil, 1)
    # each sampled output's four convolution outputs as one 2x2 plane, through O5
    quads = pts.reshape(2, 2, -1).transpose(2, 0, 1)[None]
    ref = oracle.relu_pool(quads, relu=True, pool=True).reshape(-1)
    check(got_all[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]], ref, "sampled")


def test_empty_batch():
    L = RESNET.replace(N=0)
    xd = torch.empty(L.x_shape, dtype=torch.float16, device="cuda")
    wd = torch.zeros(L.w_shape, dtype=torch.float16, device="cuda")
    y = ciw.conv2d(xd, wd, None, 1, 1, flags=IMP)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, 64, 56, 56)


def test_errors():
    def st(flags, dtype=torch.float16, C=64, W=56, sh=1, groups=1, ws_bytes=None):
        x = torch.zeros((1, C, 8, W), dtype=dtype, device="cuda")
        w = torch.zeros((C if groups > 1 else 64, C // groups, 3, 3), dtype=dtype, device="cuda")
        desc = ciw.make_desc(x.shape, w.shape, (sh, 1), 1, 1, groups)
        P, Q = ciw.conv2d_output_dims(desc, flags)
        y = torch.empty((1, w.shape[0], P, Q), dtype=dtype, device="cuda")
        ws = torch.empty(ws_bytes or (1 << 20), dtype=torch.uint8, device="cuda")
        fn = ciw._lib.load().conv2d_dw_fwd if groups > 1 else ciw._lib.load().conv2d_fwd
        import ctypes
        code = {torch.float16: ciw.CIW_F16, torch.float32: ciw.CIW_F32}[dtype]
        return fn(ctypes.byref(desc), code, code, x.data_ptr(), w.data_ptr(), None, y.data_ptr(),
                  ws.data_ptr(), ws.numel(), flags, None)
    assert st(IMP) == 0
    assert st(IMP | ciw.CIW_FLAG_MAXPOOL2) == 0
    assert st(IMP, C=24) == ciw._lib.CIW_ERR_UNSUPPORTED
    assert st(IMP, W=52) == ciw._lib.CIW_ERR_UNSUPPORTED
    assert st(IMP, sh=2) == ciw._lib.CIW_ERR_UNSUPPORTED
    assert st(IMP, dtype=torch.float32) == 0             # fp32: the matrix-core in-LDS form
    assert st(IMP | ciw.CIW_FLAG_MAXPOOL2, dtype=torch.float32) == ciw._lib.CIW_ERR_UNSUPPORTED
    assert st(IMP | ciw.CIW_FLAG_WINDOW_READY) == ciw._lib.CIW_ERR_INVALID_ARG
    assert st(IMP | ciw.CIW_FLAG_GENERIC) == ciw._lib.CIW_ERR_INVALID_ARG
    assert st(IMP, groups=64) == 0                       # depthwise: windows in LDS too
    # the band kernel (3x3, no pool) needs no workspace; the pooled call runs
    # the row-band kernel, whose re-laid-out filter does not fit in 1 KB
    assert st(IMP, ws_bytes=16) == 0
    assert st(IMP | ciw.CIW_FLAG_MAXPOOL2, ws_bytes=1024) == ciw._lib.CIW_ERR_WORKSPACE
    torch.cuda.synchronize()


# ------------------------------------------------------------ fp32 dense
from tests.test_fp32_m16_model import plan as m16_plan  # noqa: E402
MID = workloads.LAYERS["mid_3x3_fp32"]


def run_materialised_matrix(L, x, w, b, relu=False):
    """The same layer through the window tensor, the fp32 matrix-core kernel forced."""
    flags = ciw.CIW_FLAG_FP32_MFMA | (ciw.CIW_FLAG_RELU if relu else 0)
    return run(L, x, w, b, flags=flags)


@pytest.mark.parametrize("relu", [False, True])
def test_mid_layer_fp32_in_lds_every_output(relu):
    """The 1x512x13x13 -> 1024 layer in full: every output against the
    oracle, and bit for bit against the materialised path on the same
    kernel (the whole-sum kernel both ways: same products, same order)."""
    L = MID
    say(f"fp32 in-LDS: {L.name} relu={relu}")
    x, w, b = workloads.make_inputs(L)
    flags = IMP | (ciw.CIW_FLAG_RELU if relu else 0)
    y = run(L, x, w, b, flags=flags)
    got = to_host_f64(y)
    ref = oracle.conv2d(f64(x, "f32"), f64(w, "f32"), f64(b, "f32"), L.stride, L.pad, L.dil, 1)
    if relu:
        ref = oracle.relu_pool(ref, relu=True, pool=False)
    e = rel_err(got, ref)
    say(f"  rel err {e:.3e}")
    assert got.shape == ref.shape and np.all(np.isfinite(got)) and e <= TOL["f32"]
    ym = run_materialised_matrix(L, x, w, b, relu=relu)
    assert torch.equal(y, ym)


FP32_SHAPES = [
    # N, C, H, W, K, R, stride, pad, dil
    (1, 16, 32, 32, 32, 3, 1, 1, 1),       # the 1x16x32x32 -> 32 layer's geometry: several pixel blocks
    (2, 20, 9, 11, 5, 3, (2, 1), 0, 1),    # stride_h 2, ragged last chunk, K < 32
    (1, 18, 10, 12, 40, 3, (1, 2), 2, 2),  # stride_w 2, dilation 2, padding 2, K not a multiple of 32
    (3, 33, 7, 7, 70, 1, 1, 0, 1),         # 1x1, odd C
    (2, 64, 8, 56, 64, 3, 1, 1, 1),        # three pixel blocks of 3 rows
    (1, 48, 5, 100, 8, 3, 1, 1, 1),        # 100-pixel rows: one row a block
    (1, 12, 10, 12, 16, 3, (1, 2), 2, 2),  # whole-sum kernel in LDS: stride_w 2, dilation 2, 13 staged rows
]


@pytest.mark.parametrize("shape", FP32_SHAPES)
def test_fp32_in_lds_shapes_against_oracle(shape):
    N, C, H, W, K, R, stride, pad, dil = shape
    L = MID.replace(name="fp32_shape", N=N, C=C, H=H, W=W, K=K, R=R, S=R,
                    stride=stride if isinstance(stride, tuple) else (stride, stride),
                    pad=(pad, pad), dil=(dil, dil), seed=sum(shape[:6]))
    say(f"fp32 in-LDS shape {shape}")
    x, w, b = workloads.make_inputs(L)
    got = to_host_f64(run(L, x, w, b))
    ref = oracle.conv2d(f64(x, "f32"), f64(w, "f32"), f64(b, "f32"), L.stride, L.pad, L.dil, 1)
    e = rel_err(got, ref)
    say(f"  rel err {e:.3e}")
    assert got.shape == ref.shape and np.all(np.isfinite(got)) and e <= TOL["f32"]
    # where the whole-sum kernel runs the layer both ways, the in-LDS form
    # equals the materialised one bit for bit (same products, same order)
    sh, sw = L.stride
    both = all(m16_plan(N, C, H, W, K, R, R, sh, sw, pad, pad, dil, dil, imp=v) is not None
               for v in (False, True))
    if both:
        y_imp = run(L, x, w, b)
        assert torch.equal(y_imp, run_materialised_matrix(L, x, w, b))


def test_fp32_in_lds_workspace():
    """The mid layer runs through the whole-sum kernel: no workspace.  A
    layer with C not a multiple of 4 takes the split kernel, whose workspace
    holds the channel slices' partial sums; too small a one is refused."""
    d = ciw.make_desc(MID.x_shape, MID.w_shape, MID.stride, MID.pad, MID.dil, 1)
    assert ciw.conv2d_implicit_workspace_bytes(d, ciw.CIW_F32, ciw.CIW_F32, IMP) == 0
    L = MID.replace(name="odd_c", C=510)
    d = ciw.make_desc(L.x_shape, L.w_shape, L.stride, L.pad, L.dil, 1)
    nbytes = ciw.conv2d_implicit_workspace_bytes(d, ciw.CIW_F32, ciw.CIW_F32, IMP)
    assert nbytes > 0 and nbytes % (1024 * 13 * 13 * 4) == 0
    x, w, b = (to_dev(a, "f32") for a in workloads.make_inputs(L))
    y = torch.empty((1, 1024, 13, 13), dtype=torch.float32, device="cuda")
    ws = torch.empty(nbytes - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(ciw.Im2winError):
        ciw.conv2d_fwd(x, w, b, y, ws, L.stride, L.pad, L.dil, flags=IMP)
    torch.cuda.synchronize()


# ------------------------------------------------------------ few input channels
STEM = workloads.LAYERS["stem_7x7_s2_bf16"]


def test_stem_full_size_every_output():
    """The 128x3x224x224 -> 64 7x7 stride-2 layer in the launch configuration
    the benchmark times (bands of 28 rows, 7 steps of 4): every output
    against the oracle, and against the materialised path."""
    L = STEM
    say("few-channel in-LDS: stem full size, every output")
    x, w, b = workloads.make_inputs(L)
    y = run(L, x, w, b)
    got = to_host_f64(y)
    ref = oracle.conv2d(f64(x, "bf16"), f64(w, "bf16"), f64(b, "bf16"), L.stride, L.pad, L.dil, 1)
    check(got, ref, "stem full size")
    explicit = to_host_f64(run(L, x, w, b, flags=0))
    check(got, explicit, "against the materialised path")


@pytest.mark.parametrize("n", [1, 24])
def test_stem_reduced_batch_every_output(n):
    """One image (bands of one row) and 24 images (bands of 5 rows: a step
    of 4 rows, then one of 1)."""
    L = STEM.replace(N=n, seed=30 + n)
    say(f"few-channel in-LDS: stem N={n}, every output")
    x, w, b = workloads.make_inputs(L)
    got = to_host_f64(run(L, x, w, b))
    ref = oracle.conv2d(f64(x, "bf16"), f64(w, "bf16"), f64(b, "bf16"), L.stride, L.pad, L.dil, 1)
    check(got, ref, f"N={n}")


# (N, C, H, W, K, R, S, stride, pad, dil_h): filter halves, ragged blocks and
# steps, both strip alignments (d = 0, 1), trailing-entry masks, stride and
# dilation, and each store form (staged runs, 4-pixel runs, single pixels)
NARROW_SHAPES = [
    (2, 3, 23, 40, 40, 7, 7, (2, 2), (3, 3), 1),    # Q = 20: 4-pixel stores for 16-bit outputs
    (1, 2, 30, 64, 24, 5, 5, (1, 2), (2, 1), 1),    # 5x5 (a trailing entry masked), K <= 32
    (1, 4, 26, 32, 33, 5, 6, (3, 2), (1, 1), 2),    # S = 6, stride_h 3, dil_h 2, Q = 15: single pixels
    (1, 1, 17, 16, 8, 7, 7, (2, 4), (0, 3), 1),     # one channel, stride_w 4, no row padding
    (2, 3, 12, 8, 64, 3, 7, (2, 2), (1, 5), 1),     # pad_w 5 (L = 8), 9 pairs: the 6-step form
    (40, 3, 64, 64, 64, 7, 7, (2, 2), (3, 3), 1),   # bands of 3 rows (the last of 2), 32-pixel rows
    (128, 3, 64, 256, 48, 7, 7, (2, 2), (3, 3), 1),  # bands of 8 rows: two steps of 4 through the ring
]


@pytest.mark.parametrize("shape", NARROW_SHAPES)
@pytest.mark.parametrize("dtype,out", [("bf16", "bf16"), ("f16", "f16"), ("bf16", "f32"), ("f16", "f32")])
def test_narrow_shapes_against_oracle(shape, dtype, out):
    N, C, H, W, K, R, S, stride, pad, dh = shape
    L = STEM.replace(name="narrow", N=N, C=C, H=H, W=W, K=K, R=R, S=S, stride=stride, pad=pad,
                     dil=(dh, 1), dtype=dtype, out_dtype=out, x_dist=("normal", 0.0, 1.0),
                     b_dist=("uniform", -0.1, 0.1), seed=sum(shape[:7]))
    say(f"few-channel in-LDS {shape} {dtype}->{out}")
    x, w, b = workloads.make_inputs(L)
    got = to_host_f64(run(L, x, w, b))
    ref = oracle.conv2d(f64(x, dtype), f64(w, dtype), f64(b, dtype), L.stride, L.pad, L.dil, 1)
    check(got, ref, f"{shape} {dtype}->{out}")


def test_stem_relu_no_bias():
    L = STEM.replace(N=3, seed=41)
    x, w, _ = workloads.make_inputs(L)
    got = to_host_f64(run(L, x, w, None, flags=IMP | ciw.CIW_FLAG_RELU))
    conv = oracle.conv2d(f64(x, "bf16"), f64(w, "bf16"), None, L.stride, L.pad, L.dil, 1)
    check(got, oracle.relu_pool(conv, relu=True, pool=False), "relu")
    assert np.all(got >= 0)


def test_stem_non_finite_inputs_stay_in_their_windows():
    """Infinities and a NaN in x reach exactly the outputs whose windows
    hold them: a strip's entries from other windows are masked, so they
    never meet a zero filter tap (0 x Inf)."""
    L = STEM.replace(N=2, H=40, W=48, seed=43)
    x, w, b = workloads.make_inputs(L)
    x = x.copy()
    # bf16 bit patterns: +Inf, -Inf, +Inf, NaN
    for (n, c, h, col), v in (((0, 0, 3, 10), 0x7F80), ((0, 1, 17, 33), 0xFF80),
                              ((1, 2, 39, 47), 0x7F80), ((1, 1, 0, 0), 0x7FC0)):
        x[n, c, h, col] = v
    got = to_host_f64(run(L, x, w, b))
    ref = oracle.conv2d(f64(x, "bf16"), f64(w, "bf16"), f64(b, "bf16"), L.stride, L.pad, L.dil, 1)
    assert (~np.isfinite(ref)).sum() > 0
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    np.testing.assert_array_equal(np.isinf(got), np.isinf(ref))
    np.testing.assert_array_equal(np.sign(got[np.isinf(got)]), np.sign(ref[np.isinf(ref)]))
    fin = np.isfinite(ref)
    assert rel_err(got[fin], ref[fin]) <= TOL["f16"]


def test_stem_flags_and_workspace():
    """No workspace; the fused pool is refused (UNSUPPORTED) rather than
    run through the materialised path."""
    d = ciw.make_desc(STEM.x_shape, STEM.w_shape, STEM.stride, STEM.pad, STEM.dil, 1)
    for out in (ciw.CIW_BF16, ciw.CIW_F32):
        assert ciw.conv2d_implicit_workspace_bytes(d, ciw.CIW_BF16, out, IMP) == 0
        assert ciw.conv2d_implicit_workspace_bytes(d, ciw.CIW_BF16, out, IMP | ciw.CIW_FLAG_RELU) == 0
    with pytest.raises(ciw.Im2winError):
        ciw.conv2d_implicit_workspace_bytes(d, ciw.CIW_BF16, ciw.CIW_BF16, IMP | ciw.CIW_FLAG_MAXPOOL2)


# ------------------------------------------------------------ depthwise
DW = workloads.LAYERS["dw_3x3_fp32"]


def run_dw(L, x, w, b, flags=IMP):
    od = torch_dtype(L.out_dtype)
    y = ciw.conv2d(to_dev(x, L.dtype), to_dev(w, L.dtype), to_dev(b, L.dtype), L.stride, L.pad,
                   L.dil, L.groups, out_dtype=od, flags=flags)
    torch.cuda.synchronize()
    return y


def test_dw_layer_full_size_sampled():
    """The 128x512x14x14 depthwise layer at full size: sampled outputs
    against the oracle, every output against the materialised path."""
    L = DW
    say("implicit dw_3x3_fp32 full size, sampled")
    x, w, b = workloads.make_inputs(L)
    got = to_host_f64(run_dw(L, x, w, b))
    rng = np.random.default_rng(93)
    idx = sample_indices(got.shape, 3000, rng)
    f = lambda a: a.astype(np.float64)
    ref = oracle.conv2d_points(f(x), f(w), f(b), idx, L.stride, L.pad, L.dil, L.groups)
    e = rel_err(got[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]], ref)
    say(f"  sampled: rel err {e:.3e}")
    assert e <= TOL["f32"]
    explicit = to_host_f64(run_dw(L, x, w, b, flags=0))
    e = rel_err(got, explicit)
    say(f"  against the materialised path: rel err {e:.3e}")
    assert e <= TOL["f32"] and np.all(np.isfinite(got))


# (N, C, H, W, R, stride, pad, dil, dtype, out)
DW_SHAPES = [
    (2, 512, 14, 14, 3, 1, 1, 1, "f32", "f32"),
    (3, 7, 9, 11, 3, 2, 1, 1, "f32", "f32"),
    (2, 5, 17, 13, 5, 1, 2, 2, "f16", "f16"),
    (1, 9, 30, 30, 7, 2, 3, 1, "bf16", "bf16"),
    (2, 6, 12, 10, 3, 1, 0, 1, "f16", "f32"),
    (1, 3, 64, 64, 3, 1, 1, 1, "bf16", "f32"),
    (4, 33, 1, 1, 1, 1, 0, 1, "f32", "f32"),
    (1, 4, 70, 70, 3, 1, 1, 1, "f32", "f32"),    # 16-byte staging, a plane over two load rounds
    (2, 10, 6, 6, 5, 2, 2, 1, "f32", "f32"),     # 16-byte staging, float4s across row ends
]


@pytest.mark.parametrize("shape", DW_SHAPES)
@pytest.mark.parametrize("epi", ["none", "relu", "relu_pool"])
def test_dw_shapes_against_oracle(shape, epi):
    N, C, H, W, R, s, p, d, dt, out = shape
    L = workloads.Layer("dwimp", N=N, C=C, H=H, W=W, K=C, R=R, S=R, stride=(s, s), pad=(p, p),
                        dil=(d, d), groups=C, dtype=dt, out_dtype=out,
                        x_dist=("normal", 0.0, 1.0), seed=sum(shape[:8]))
    P = (H + 2 * p - d * (R - 1) - 1) // s + 1
    if epi == "relu_pool" and P < 2:
        pytest.skip("no 2x2 region")
    say(f"implicit dw {shape} {epi}")
    x, w, b = workloads.make_inputs(L)
    flags = IMP | {"none": 0, "relu": ciw.CIW_FLAG_RELU,
                   "relu_pool": ciw.CIW_FLAG_RELU | ciw.CIW_FLAG_MAXPOOL2}[epi]
    got = to_host_f64(run_dw(L, x, w, b, flags))
    ref = oracle.conv2d(f64(x, dt), f64(w, dt), f64(b, dt), L.stride, L.pad, L.dil, L.groups)
    if epi != "none":
        ref = oracle.relu_pool(ref, relu=True, pool=epi == "relu_pool")
    e = rel_err(got, ref)
    say(f"  rel err {e:.3e}")
    assert got.shape == ref.shape and np.all(np.isfinite(got))
    assert e <= TOL[dt]

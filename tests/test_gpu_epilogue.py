"""GPU parity of the fused epilogue (bias, ReLU, 2x2 max-pool) on every path.

The conv -> scale/bias -> max-pool chain of the CS149 page ("Fusion: keep
intermediates out of memory") runs inside the contraction kernels when
CIW_FLAG_RELU / CIW_FLAG_MAXPOOL2 are set.  Each test compares the result
with the oracle's convolution followed by its epilogue (O5), to the same
tolerance as the plain convolution: the max is 1-Lipschitz, so a pooled
output is off by at most its region's largest error.  Every kernel that
carries the epilogue is reached: the matrix-core row kernel in each of its
layouts, the generic matrix-core kernel, the fp32 vector kernel with the
channel sum in one pass (pool in registers) and split (pool in the split
reduction), the generic fp32 kernel, and the depthwise block and generic
kernels; odd output extents check that the last row and column are dropped.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from tests import row_kernel_cases
from tests.gpu_util import TOL, rel_err, to_dev, to_host_bits, to_host_f64, torch_dtype

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import cnn_convolution_im2win_amd as ciw  # noqa: E402

CODE = {"f32": ciw.CIW_F32, "f16": ciw.CIW_F16, "bf16": ciw.CIW_BF16}
RELU, POOL = ciw.CIW_FLAG_RELU, ciw.CIW_FLAG_MAXPOOL2
EPILOGUES = {"relu": RELU, "pool": POOL, "relu_pool": RELU | POOL}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(L, a):
    return None if a is None else workloads.to_f64(a, L.dtype)


def reference(L, x, w, b, flags):
    y = oracle.conv2d(f64(L, x), f64(L, w), f64(L, b), L.stride, L.pad, L.dil, L.groups)
    return oracle.relu_pool(y, relu=bool(flags & RELU), pool=bool(flags & POOL))


def run(L, x, w, b, flags, out_dtype=None, workspace_images=None):
    desc = ciw.make_desc(L.x_shape, L.w_shape, L.stride, L.pad, L.dil, L.groups)
    ws = None
    if workspace_images is not None:
        nbytes = ciw.conv2d_workspace_bytes(desc, CODE[L.dtype], workspace_images)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    y = ciw.conv2d(to_dev(x, L.dtype), to_dev(w, L.dtype), to_dev(b, L.dtype), L.stride, L.pad,
                   L.dil, L.groups, out_dtype=torch_dtype(out_dtype or L.out_dtype),
                   workspace=ws, flags=flags)
    torch.cuda.synchronize()
    return y


def check(L, x, w, b, flags, what, extra=0, out_dtype=None):
    ref = reference(L, x, w, b, flags)
    got = to_host_f64(run(L, x, w, b, flags | extra, out_dtype))
    od = out_dtype or L.out_dtype
    tol = TOL["f32"] if od == "f32" else TOL[L.dtype]
    e = rel_err(got, ref)
    say(f"  {what}: rel err {e:.3e} (tol {tol:.0e})")
    assert got.shape == ref.shape, what
    assert np.all(np.isfinite(got)), what
    if flags & RELU:
        assert np.all(got >= 0), what
    assert e <= tol, what


def pooled_points(L, x, w, b, idx, relu):
    """O5 at pooled indices (n, k, j, i): O1 at the region's four pixels."""
    pts = []
    for dy in (0, 1):
        for dx in (0, 1):
            q = idx.copy()
            q[:, 2] = 2 * idx[:, 2] + dy
            q[:, 3] = 2 * idx[:, 3] + dx
            pts.append(oracle.conv2d_points(f64(L, x), f64(L, w), f64(L, b), q, L.stride,
                                            L.pad, L.dil, L.groups))
    v = np.stack(pts)                       # [4, npts]
    if relu:
        v = np.fmax(v, 0.0)
    return np.fmax.reduce(v, axis=0)


# ------------------------------------------------------------ matrix cores
@pytest.mark.parametrize("epi", list(EPILOGUES))
@pytest.mark.parametrize("name", list(row_kernel_cases.CASES))
def test_row_kernel_layouts(name, epi):
    L = row_kernel_cases.CASES[name]
    say(f"row kernel {name} {epi}: x{L.x_shape} w{L.w_shape} s={L.stride} p={L.pad} "
        f"{L.dtype}->{L.out_dtype}")
    x, w, b = workloads.make_inputs(L)
    check(L, x, w, b, EPILOGUES[epi], f"{name} {epi}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_generic_matrix_core_kernel(dtype):
    # K > 64 and a dilated layer leave the row kernel; GENERIC forces it
    rng = np.random.default_rng(41)
    layers = [workloads.Layer("k80", N=2, C=12, H=11, W=13, K=80, R=3, S=3, pad=(1, 1),
                              dtype=dtype, out_dtype=dtype, x_dist=("normal", 0.0, 1.0),
                              w_dist=("he_normal",), b_dist=("uniform", -0.5, 0.5), seed=5),
              workloads.Layer("dil", N=1, C=8, H=15, W=14, K=24, R=3, S=3, stride=(1, 2),
                              pad=(2, 1), dil=(1, 2), dtype=dtype, out_dtype=dtype,
                              x_dist=("normal", 0.0, 1.0), w_dist=("he_normal",), b_dist=None,
                              seed=6)]
    layers += [workloads.random_layer(rng, dtype=dtype, max_hw=16, max_c=24, max_k=48)
               for _ in range(6)]
    for i, L in enumerate(layers):
        P, Q = oracle.out_dims(L.x_shape, L.w_shape, L.stride, L.pad, L.dil)
        if P < 2 or Q < 2:
            continue
        x, w, b = workloads.make_inputs(L)
        say(f"generic mfma #{i} x{L.x_shape} w{L.w_shape} P,Q={P},{Q}")
        for epi, fl in EPILOGUES.items():
            check(L, x, w, b, fl, f"#{i} {epi}", extra=ciw.CIW_FLAG_GENERIC)
            if i < 2:
                check(L, x, w, b, fl, f"#{i} {epi} default path")


@pytest.mark.parametrize("name", ["resnet_3x3_fp16", "stem_7x7_s2_bf16"])
def test_full_size_pooled_sampled(name):
    # the full batch in the configuration the benchmark times, pooled and
    # rectified; sampled outputs against the oracle one region at a time
    L = workloads.LAYERS[name]
    say(f"{name} full size, relu + pool, sampled")
    x, w, b = workloads.make_inputs(L)
    y = to_host_f64(run(L, x, w, b, RELU | POOL))
    P, Q = oracle.out_dims(L.x_shape, L.w_shape, L.stride, L.pad, L.dil)
    assert y.shape == (L.N, L.K, P // 2, Q // 2)
    assert np.all(np.isfinite(y)) and np.all(y >= 0)
    rng = np.random.default_rng(78)
    idx = np.stack([rng.integers(0, s, size=600) for s in y.shape], axis=1).astype(np.int64)
    corners = [(n, k, j, i) for n in (0, L.N - 1) for k in (0, L.K - 1)
               for j in (0, y.shape[2] - 1) for i in (0, y.shape[3] - 1)]
    idx = np.concatenate([idx, np.array(corners, dtype=np.int64)])
    ref = pooled_points(L, x, w, b, idx, relu=True)
    got = y[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3]]
    e = rel_err(got, ref)
    say(f"  sampled rel err {e:.3e}")
    assert e <= TOL[L.dtype]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_half_inputs_fp32_output_pooled(dtype):
    L = workloads.LAYERS["resnet_3x3_fp16"].replace(N=1, H=19, W=21, dtype=dtype,
                                                    out_dtype="f32",
                                                    b_dist=("uniform", -0.1, 0.1))
    x, w, b = workloads.make_inputs(L)
    check(L, x, w, b, RELU | POOL, f"{dtype}->f32 relu+pool")


# ------------------------------------------------------------ fp32 vector ALUs
@pytest.mark.parametrize("epi", list(EPILOGUES))
@pytest.mark.parametrize("flags", [0, ciw.CIW_FLAG_NO_SPLIT, ciw.CIW_FLAG_GENERIC],
                         ids=["split", "no_split", "generic"])
def test_fp32_mid_layer(flags, epi):
    # 13 x 13: the pool drops row and column 12
    L = workloads.LAYERS["mid_3x3_fp32"]
    say(f"mid fp32 {epi} flags {flags}")
    x, w, b = workloads.make_inputs(L)
    check(L, x, w, b, EPILOGUES[epi], f"mid {epi} flags {flags}", extra=flags)


@pytest.mark.parametrize("flags", [0, ciw.CIW_FLAG_NO_SPLIT, ciw.CIW_FLAG_GENERIC],
                         ids=["split", "no_split", "generic"])
def test_fp32_random_layers(flags):
    rng = np.random.default_rng(42)
    for i in range(16):
        L = workloads.random_layer(rng, dtype="f32", max_hw=22, max_c=40, max_k=80)
        P, Q = oracle.out_dims(L.x_shape, L.w_shape, L.stride, L.pad, L.dil)
        if P < 2 or Q < 2:
            continue
        x, w, b = workloads.make_inputs(L)
        fl = list(EPILOGUES.values())[i % 3]
        say(f"fp32 #{i} x{L.x_shape} w{L.w_shape} s={L.stride} P,Q={P},{Q} flags {fl}")
        check(L, x, w, b, fl, f"fp32 #{i}", extra=flags)


def test_fp32_tiny_layer_batch():
    L = workloads.LAYERS["tiny_3x3_fp32"].replace(N=3, H=31, W=30)
    x, w, b = workloads.make_inputs(L)
    for epi, fl in EPILOGUES.items():
        check(L, x, w, b, fl, f"tiny {epi}")


# ------------------------------------------------------------ depthwise
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_depthwise_layers(dtype):
    # odd P: pooled rows skip a window row at every plane boundary
    base = workloads.LAYERS["dw_3x3_fp32"]
    layers = [base.replace(N=2, dtype=dtype, out_dtype=dtype),
              base.replace(N=2, C=40, K=40, groups=40, H=13, W=15, dtype=dtype, out_dtype=dtype),
              base.replace(N=1, C=24, K=24, groups=24, H=23, W=9, R=5, S=5, pad=(2, 2),
                           dtype=dtype, out_dtype=dtype),
              base.replace(N=1, C=8, K=8, groups=8, H=17, W=19, R=7, S=7, pad=(3, 3),
                           stride=(2, 2), dtype=dtype, out_dtype=dtype)]
    for i, L in enumerate(layers):
        x, w, b = workloads.make_inputs(L)
        say(f"depthwise #{i} {dtype} x{L.x_shape} R,S={L.R},{L.S} s={L.stride}")
        for epi, fl in EPILOGUES.items():
            for extra in (0, ciw.CIW_FLAG_GENERIC):
                check(L, x, w, b, fl, f"dw #{i} {epi} extra {extra}", extra=extra)


def test_depthwise_random_layers():
    rng = np.random.default_rng(43)
    for i in range(12):
        dtype = ("f32", "f16", "bf16")[i % 3]
        L = workloads.random_layer(rng, dtype=dtype, depthwise=True, max_hw=24, max_c=40)
        P, Q = oracle.out_dims(L.x_shape, L.w_shape, L.stride, L.pad, L.dil)
        if P < 2 or Q < 2:
            continue
        x, w, b = workloads.make_inputs(L)
        fl = list(EPILOGUES.values())[i % 3]
        say(f"dw random #{i} {dtype} x{L.x_shape} R,S={L.R},{L.S} P,Q={P},{Q} flags {fl}")
        check(L, x, w, b, fl, f"dw random #{i}")


# ------------------------------------------------------------ chunking
@pytest.mark.parametrize("name", ["resnet_3x3_fp16", "stem_7x7_s2_bf16", "dw_3x3_fp32",
                                  "mid_3x3_fp32"])
def test_chunked_pooled_equals_full_batch(name):
    # batch chunks write pooled outputs at pooled image offsets
    L = workloads.LAYERS[name]
    L = L.replace(N=min(L.N, 3))
    say(f"chunked relu+pool {name} N={L.N}")
    x, w, b = workloads.make_inputs(L)
    full = run(L, x, w, b, RELU | POOL)
    for imgs in (1, 2):
        part = run(L, x, w, b, RELU | POOL, workspace_images=imgs)
        if L.dtype == "f32" and L.groups == 1:
            # the fp32 channel split depends on the chunk size
            check(L, x, w, b, RELU | POOL, f"{name} chunk {imgs}")
        else:
            assert np.array_equal(to_host_bits(part), to_host_bits(full)), f"{name} chunk {imgs}"

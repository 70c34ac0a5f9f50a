"""Pins for the CPU oracle (no GPU).

Every check here ties the oracle to something other than itself: closed
forms worked out by hand, scipy's 2-D cross-correlation, a numpy im2col
product, textbook reductions (1x1 conv = matrix product, full-size filter =
fully connected layer), invariants (delta filter, linearity, zero-padding tap
counts) and the diagonalwise identity for depthwise layers.  The fused
epilogue (ReLU, 2x2 max-pool) is pinned by closed forms on ramps, torch's
CPU max_pool2d, the ReLU/max commutation and IEEE maxNum on NaN.
"""
import numpy as np
import pytest
from scipy import signal

import oracle
import workloads

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def ramp16():
    # X = 1..16 as a 1x1x4x4 image: X[i][j] = 4i + j + 1
    return np.arange(1, 17, dtype=np.float64).reshape(1, 1, 4, 4)


# ---------------------------------------------------------------- closed forms
def test_all_ones_3x3_valid_closed_form():
    # Window sum of X[i][j] = 4i+j+1 over rows i..i+2, cols j..j+2:
    # 9 * (4(i+1) + (j+1) + 1) = 36 i + 9 j + 54.
    y = oracle.conv2d(ramp16(), np.ones((1, 1, 3, 3)))
    expect = np.array([[36 * i + 9 * j + 54 for j in range(2)] for i in range(2)])
    assert y.shape == (1, 1, 2, 2)
    assert np.array_equal(y[0, 0], expect)          # [[54, 63], [90, 99]]


def test_ramp_filter_pins_cross_correlation():
    # F[r][q] = 3r + q + 1.  At (0,0): sum (3r+q+1)(4r+q+1) = 14 + 92 + 242 = 348.
    # Shifting the window by (i, j) adds 4i+j to each input, and sum(F) = 45,
    # so Y(i,j) = 348 + 45 (4i + j).  A flipped filter (convolution) would give
    # sum (9-3r-q)(4r+q+1) = 192 at (0,0).
    f = np.arange(1, 10, dtype=np.float64).reshape(1, 1, 3, 3)
    y = oracle.conv2d(ramp16(), f)
    expect = np.array([[348 + 45 * (4 * i + j) for j in range(2)] for i in range(2)])
    assert np.array_equal(y[0, 0], expect)          # [[348, 393], [528, 573]]
    assert y[0, 0, 0, 0] != 192
    yb = oracle.conv2d(ramp16(), f, b=np.array([0.5]))
    assert np.array_equal(yb[0, 0], expect + 0.5)


def test_stride2_pad1_closed_form():
    # stride 2, pad 1 on the 4x4 ramp: outputs at (0,0),(0,2),(2,0),(2,2) of the
    # pad-1 stride-1 result; window sums over the in-bounds part.
    y = oracle.conv2d(ramp16(), np.ones((1, 1, 3, 3)), stride=2, pad=1)
    X = ramp16()[0, 0]
    # (0,0): rows 0..1, cols 0..1 -> 1+2+5+6 = 14;  (0,1): rows 0..1, cols 1..3
    # -> 2+3+4+6+7+8 = 30; (1,0): rows 1..3, cols 0..1 -> 5+6+9+10+13+14 = 57;
    # (1,1): rows 1..3, cols 1..3 -> 99 (the interior window sum from above).
    assert np.array_equal(y[0, 0], np.array([[14, 30], [57, 99]]))
    assert X[0:2, 0:2].sum() == 14


def test_dilation2_closed_form():
    # 2x2 all-ones filter dilated by 2 samples X[i][j], X[i][j+2], X[i+2][j],
    # X[i+2][j+2]: 4 (4i+j+1) + (0 + 2 + 8 + 10) = 16 i + 4 j + 24.
    y = oracle.conv2d(ramp16(), np.ones((1, 1, 2, 2)), dil=2)
    expect = np.array([[16 * i + 4 * j + 24 for j in range(2)] for i in range(2)])
    assert np.array_equal(y[0, 0], expect)          # [[24, 28], [40, 44]]


def test_zero_padding_tap_counts():
    # All-ones input and filter, 3x3, pad 1: each output counts the in-bounds
    # taps times C -- corners 4C, edges 6C, interior 9C.
    C = 2
    y = oracle.conv2d(np.ones((1, C, 5, 6)), np.ones((1, C, 3, 3)), pad=1)[0, 0]
    assert y[0, 0] == y[0, -1] == y[-1, 0] == y[-1, -1] == 4 * C
    assert np.all(y[0, 1:-1] == 6 * C) and np.all(y[-1, 1:-1] == 6 * C)
    assert np.all(y[1:-1, 0] == 6 * C) and np.all(y[1:-1, -1] == 6 * C)
    assert np.all(y[1:-1, 1:-1] == 9 * C)


@pytest.mark.parametrize("H,R,s,p,d,P", [
    (13, 3, 1, 1, 1, 13),    # the OpenCL-Benchmarks layer: 13 -> 13
    (224, 7, 2, 3, 1, 112),  # 7x7 stride-2 stem: 224 -> 112
    (56, 3, 1, 1, 1, 56), (32, 3, 1, 1, 1, 32), (14, 3, 1, 1, 1, 14),
    (4, 3, 1, 0, 1, 2), (4, 2, 1, 0, 2, 2), (5, 5, 3, 0, 1, 1),
])
def test_output_extent(H, R, s, p, d, P):
    # brute-force count of window start positions that fit the padded input
    count = sum(1 for st in range(0, H + 2 * p, s) if st + d * (R - 1) < H + 2 * p)
    assert count == P
    assert oracle.out_dims((1, 1, H, H), (1, 1, R, R), s, p, d) == (P, P)


# ---------------------------------------------------------------- library routines
def scipy_conv(x, w, b, stride, pad, dil, groups):
    """Reference built on scipy.signal.correlate2d: zero-pad, correlate with the
    zero-dilated filter in 'valid' mode, subsample by the stride."""
    N, C, H, W = x.shape
    K, Cg, R, S = w.shape
    (sh, sw), (ph, pw), (dh, dw) = stride, pad, dil
    Kg = K // groups
    out = None
    for n in range(N):
        for k in range(K):
            g = k // Kg
            acc = 0.0
            for c in range(Cg):
                fd = np.zeros((dh * (R - 1) + 1, dw * (S - 1) + 1))
                fd[::dh, ::dw] = w[k, c]
                xp = np.pad(x[n, g * Cg + c], ((ph, ph), (pw, pw)))
                acc = acc + signal.correlate2d(xp, fd, mode="valid")
            acc = acc[::sh, ::sw]
            if b is not None:
                acc = acc + b[k]
            if out is None:
                out = np.zeros((N, K) + acc.shape)
            out[n, k] = acc
    return out


def test_against_scipy_correlate2d_random():
    rng = np.random.default_rng(123)
    for _ in range(25):
        L = workloads.random_layer(rng, max_hw=9, max_c=4, max_k=4)
        x, w, b = (None if a is None else workloads.to_f64(a, L.dtype)
                   for a in workloads.make_inputs(L))
        y = oracle.conv2d(x, w, b, L.stride, L.pad, L.dil, L.groups)
        ref = scipy_conv(x, w, b, L.stride, L.pad, L.dil, L.groups)
        assert y.shape == ref.shape, L
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_against_scipy_depthwise_random():
    rng = np.random.default_rng(7)
    for _ in range(10):
        L = workloads.random_layer(rng, depthwise=True, max_hw=9, max_c=5)
        x, w, b = (None if a is None else workloads.to_f64(a, L.dtype)
                   for a in workloads.make_inputs(L))
        y = oracle.conv2d(x, w, b, L.stride, L.pad, L.dil, L.groups)
        ref = scipy_conv(x, w, b, L.stride, L.pad, L.dil, L.groups)
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_against_numpy_im2col_random():
    rng = np.random.default_rng(99)
    for _ in range(30):
        L = workloads.random_layer(rng, max_hw=12, max_c=6, max_k=6)
        x, w, b = (None if a is None else workloads.to_f64(a, L.dtype)
                   for a in workloads.make_inputs(L))
        y = oracle.conv2d(x, w, b, L.stride, L.pad, L.dil, L.groups)
        ref = oracle.im2col_conv(x, w, b, L.stride, L.pad, L.dil, L.groups)
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_tiny_layer_against_im2col():
    L = workloads.LAYERS["tiny_3x3_fp32"]
    x, w, b = (workloads.to_f64(a, L.dtype) for a in workloads.make_inputs(L))
    y = oracle.conv2d(x, w, b, L.stride, L.pad, L.dil, L.groups)
    ref = oracle.im2col_conv(x, w, b, L.stride, L.pad, L.dil, L.groups)
    assert y.shape == (1, 32, 32, 32)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_1x1_is_matrix_product():
    rng = np.random.default_rng(5)
    x = rng.normal(size=(2, 7, 5, 6))
    w = rng.normal(size=(4, 7, 1, 1))
    y = oracle.conv2d(x, w)
    ref = np.stack([w[:, :, 0, 0] @ x[n].reshape(7, -1) for n in range(2)]).reshape(2, 4, 5, 6)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_full_size_filter_is_fully_connected():
    rng = np.random.default_rng(6)
    x = rng.normal(size=(3, 4, 5, 6))
    w = rng.normal(size=(8, 4, 5, 6))
    b = rng.normal(size=8)
    y = oracle.conv2d(x, w, b)
    assert y.shape == (3, 8, 1, 1)
    ref = x.reshape(3, -1) @ w.reshape(8, -1).T + b
    np.testing.assert_allclose(y[:, :, 0, 0], ref, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- invariants
def test_delta_filter_reproduces_input():
    rng = np.random.default_rng(8)
    for R, S in [(3, 3), (5, 3), (1, 7)]:
        C = 3
        x = rng.normal(size=(2, C, 6, 7))
        w = np.zeros((C, C, R, S))
        for c in range(C):
            w[c, c, R // 2, S // 2] = 1.0
        b = rng.normal(size=C)
        y = oracle.conv2d(x, w, b, pad=(R // 2, S // 2))
        assert np.array_equal(y, x + b[None, :, None, None])


def test_linearity():
    rng = np.random.default_rng(9)
    x1, x2 = rng.normal(size=(2, 2, 3, 7, 6))
    w1, w2 = rng.normal(size=(2, 4, 3, 3, 2))
    a, c = 0.75, -1.5
    kw = dict(stride=(2, 1), pad=(1, 2), dil=(1, 2))
    lhs = oracle.conv2d(a * x1 + c * x2, w1, **kw)
    rhs = a * oracle.conv2d(x1, w1, **kw) + c * oracle.conv2d(x2, w1, **kw)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    lhs = oracle.conv2d(x1, a * w1 + c * w2, **kw)
    rhs = a * oracle.conv2d(x1, w1, **kw) + c * oracle.conv2d(x1, w2, **kw)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    b = rng.normal(size=4)
    diff = oracle.conv2d(x1, w1, b, **kw) - oracle.conv2d(x1, w1, **kw)
    np.testing.assert_allclose(diff, np.broadcast_to(b[None, :, None, None], lhs.shape),
                               rtol=0, atol=1e-12)


def test_diagonalwise_identity():
    # "Diagonalwise Refactorization ..." (abstract): a depthwise convolution
    # equals a standard convolution whose weight matrix is diagonal in
    # (output, input) channel.  The extra terms are exact zeros, so the two
    # results are identical.
    rng = np.random.default_rng(10)
    C = 5
    x = rng.normal(size=(2, C, 7, 6))
    wdw = rng.normal(size=(C, 1, 3, 3))
    b = rng.normal(size=C)
    dense = np.zeros((C, C, 3, 3))
    for c in range(C):
        dense[c, c] = wdw[c, 0]
    for kw in [dict(pad=1), dict(stride=2, pad=(0, 1), dil=(2, 1))]:
        ydw = oracle.conv2d(x, wdw, b, groups=C, **kw)
        yd = oracle.conv2d(x, dense, b, **kw)
        assert np.array_equal(ydw, yd)


def test_points_match_full():
    rng = np.random.default_rng(11)
    L = workloads.random_layer(rng, max_hw=10, max_c=5, max_k=5)
    x, w, b = workloads.make_inputs(L)
    x, w = workloads.to_f64(x, L.dtype), workloads.to_f64(w, L.dtype)
    b = None if b is None else workloads.to_f64(b, L.dtype)
    y = oracle.conv2d(x, w, b, L.stride, L.pad, L.dil)
    idx = np.stack(np.meshgrid(*[np.arange(s) for s in y.shape], indexing="ij"), -1).reshape(-1, 4)
    pts = oracle.conv2d_points(x, w, b, idx, L.stride, L.pad, L.dil)
    assert np.array_equal(pts, y.reshape(-1))


# ---------------------------------------------------------------- im2win repack
def test_repack_worked_example_chw():
    # 4x4 ramp, 3x3 filter, stride 1, no padding: the window tensor row of
    # output row h holds input columns 0..3 in order, each as the 3 values of
    # rows h..h+2 (filter height index before width).  The window of output (0,0) is the
    # first 9 entries: columns 0..2 of rows 0..2.
    xw = oracle.im2win(ramp16(), 3, 3)
    assert xw.shape == (2, 12)              # W_win = 4 columns * 3 rows, pitch 12 (fp64: even)
    assert list(xw[0]) == [1, 5, 9, 2, 6, 10, 3, 7, 11, 4, 8, 12]
    assert list(xw[1]) == [5, 9, 13, 6, 10, 14, 7, 11, 15, 8, 12, 16]
    assert xw[0, :9].sum() == 54            # all-ones window (0,0) from the closed form
    xw = oracle.im2win(ramp16(), 3, 3, pad=1)
    assert list(xw[0, :18]) == [0, 0, 0, 0, 1, 5, 0, 2, 6, 0, 3, 7, 0, 4, 8, 0, 0, 0]


def test_repack_worked_example_two_channels():
    x = np.arange(1, 19, dtype=np.float32).reshape(1, 2, 3, 3)
    hwc = oracle.im2win(x, 2, 2, layout=oracle.LAYOUT_HWC)
    assert hwc.shape == (2, 12)
    assert list(hwc[0]) == [1, 10, 4, 13, 2, 11, 5, 14, 3, 12, 6, 15]
    assert list(hwc[1]) == [4, 13, 7, 16, 5, 14, 8, 17, 6, 15, 9, 18]
    chw = oracle.im2win(x, 2, 2, layout=oracle.LAYOUT_CHW)
    assert chw.shape == (4, 8)              # 6 elements, fp32 pitch rounds to 8
    assert list(chw[0]) == [1, 4, 2, 5, 3, 6, 0, 0]
    assert list(chw[1]) == [4, 7, 5, 8, 6, 9, 0, 0]
    assert list(chw[2]) == [10, 13, 11, 14, 12, 15, 0, 0]
    assert list(chw[3]) == [13, 16, 14, 17, 15, 18, 0, 0]


def sliding_windows(x, R, S, stride, pad, dil):
    """[N, C, P, Q, R, S] sliding windows of the zero-padded input (numpy)."""
    (sh, sw), (ph, pw), (dh, dw) = stride, pad, dil
    xp = np.pad(x, ((0, 0), (0, 0), (ph, ph), (pw, pw)))
    win = np.lib.stride_tricks.sliding_window_view(
        xp, (dh * (R - 1) + 1, dw * (S - 1) + 1), axis=(2, 3))
    return win[:, :, ::sh, ::sw, ::dh, ::dw]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_repack_windows_match_sliding_windows(dtype):
    """Every window read out of the repacked rows equals the corresponding
    im2col window of the padded input (taken column-major, i.e. height before
    width), for both layouts; pitch tails are zero; bit patterns are copied."""
    rng = np.random.default_rng(12)
    for _ in range(12):
        L = workloads.random_layer(rng, dtype=dtype, max_hw=10, max_c=5)
        x, _, _ = workloads.make_inputs(L)
        N, C, H, W = x.shape
        R, S = L.R, L.S
        win = sliding_windows(x, R, S, L.stride, L.pad, L.dil)   # bit patterns
        P, Q = win.shape[2], win.shape[3]
        sw, dw = L.stride[1], L.dil[1]
        eb = workloads.ELEM_BYTES[dtype]
        for layout in (oracle.LAYOUT_CHW, oracle.LAYOUT_HWC):
            xw = oracle.im2win(x, R, S, L.stride, L.pad, L.dil, layout)
            rows, length, pitch = oracle.window_geometry(x.shape, (1, C, R, S), layout, eb,
                                                         L.stride, L.pad, L.dil)
            assert xw.shape == (rows, pitch)
            assert (pitch * eb) % 16 == 0 and 0 <= pitch - length < 16 // eb
            assert not np.any(xw[:, length:].view(np.uint8))
            for n in range(N):
                for h in range(P):
                    for wo in range(Q):
                        for q in range(S):
                            col = wo * sw + q * dw
                            if layout == oracle.LAYOUT_CHW:
                                got = np.stack([xw[(n * C + c) * P + h, col * R:(col + 1) * R]
                                                for c in range(C)])          # [C, R]
                            else:
                                seg = xw[n * P + h, col * R * C:(col + 1) * R * C]
                                got = seg.reshape(R, C).T                    # [C, R]
                            assert np.array_equal(np.ascontiguousarray(got).view(np.uint8),
                                                  np.ascontiguousarray(win[n, :, h, wo, :, q]).view(np.uint8))


def test_repack_memory_saving_formula():
    # Im2win paper §III-B: the window tensor avoids storing the overlap of
    # horizontally adjacent windows.  Per (n, c, output row) and with dilation 1
    # the saving is R * (Q - 1) * (S - stride_w) elements, so
    # window elements (without pitch) + saving = im2col elements.  When the
    # stride equals the filter width there is no overlap and no saving.
    for (H, W, R, S, s, p) in [(13, 13, 3, 3, 1, 1), (224, 224, 7, 7, 2, 3),
                               (56, 56, 3, 3, 1, 1), (9, 11, 3, 5, 3, 0), (8, 8, 2, 2, 2, 0)]:
        N, C = 2, 3
        P, Q = oracle.out_dims((N, C, H, W), (1, C, R, S), s, p)
        _, length, _ = oracle.window_geometry((N, C, H, W), (1, C, R, S), 0, 8, s, p)
        win_elems = N * C * P * length
        im2col_elems = N * P * Q * C * R * S
        assert win_elems + N * C * P * R * (Q - 1) * (S - s) == im2col_elems
        if s == S:
            assert win_elems == im2col_elems


@pytest.mark.parametrize("layout", [oracle.LAYOUT_CHW, oracle.LAYOUT_HWC])
def test_window_conv_equals_direct(layout):
    rng = np.random.default_rng(13)
    for _ in range(20):
        L = workloads.random_layer(rng, max_hw=10, max_c=5, max_k=5)
        x, w, b = (None if a is None else workloads.to_f64(a, L.dtype)
                   for a in workloads.make_inputs(L))
        xw = oracle.im2win(x, L.R, L.S, L.stride, L.pad, L.dil, layout)
        y3 = oracle.window_conv(xw, x.shape, w, b, L.stride, L.pad, L.dil, 1, layout)
        y1 = oracle.conv2d(x, w, b, L.stride, L.pad, L.dil)
        np.testing.assert_allclose(y3, y1, rtol=1e-12, atol=1e-12)


def test_window_conv_depthwise_equals_direct():
    rng = np.random.default_rng(14)
    for _ in range(8):
        L = workloads.random_layer(rng, depthwise=True, max_hw=10, max_c=5)
        x, w, b = (None if a is None else workloads.to_f64(a, L.dtype)
                   for a in workloads.make_inputs(L))
        xw = oracle.im2win(x, L.R, L.S, L.stride, L.pad, L.dil, oracle.LAYOUT_CHW)
        y3 = oracle.window_conv(xw, x.shape, w, b, L.stride, L.pad, L.dil, L.groups)
        y1 = oracle.conv2d(x, w, b, L.stride, L.pad, L.dil, L.groups)
        np.testing.assert_allclose(y3, y1, rtol=1e-12, atol=1e-12)


# ------------------------------------------------- fused epilogue (O5)
def ramp_map(P, Q, sign=1.0):
    # y[h][w] = sign * (h Q + w) for one image and channel
    return sign * np.arange(P * Q, dtype=np.float64).reshape(1, 1, P, Q)


def test_pool_increasing_ramp_takes_bottom_right():
    # odd extents: the last row and column belong to no 2x2 region
    out = oracle.relu_pool(ramp_map(5, 7), relu=False, pool=True)
    assert out.shape == (1, 1, 2, 3)
    expect = [[(2 * j + 1) * 7 + 2 * i + 1 for i in range(3)] for j in range(2)]
    assert np.array_equal(out[0, 0], expect)


def test_pool_decreasing_ramp_takes_top_left():
    out = oracle.relu_pool(ramp_map(4, 6, -1.0), relu=False, pool=True)
    expect = [[-(2 * j * 6 + 2 * i) for i in range(3)] for j in range(2)]
    assert np.array_equal(out[0, 0], expect)


def test_relu_closed_form():
    y = np.array([-2.0, -0.5, 0.0, 0.5, 3.0]).reshape(1, 1, 1, 5)
    assert np.array_equal(oracle.relu_pool(y, relu=True, pool=False)[0, 0, 0],
                          [0.0, 0.0, 0.0, 0.5, 3.0])
    assert np.array_equal(oracle.relu_pool(y, relu=False, pool=False), y)
    # a region of negatives pools to its largest value, or to 0 after ReLU
    neg = ramp_map(2, 2, -1.0) - 1.0
    assert oracle.relu_pool(neg, relu=False, pool=True)[0, 0, 0, 0] == -1.0
    assert oracle.relu_pool(neg, relu=True, pool=True)[0, 0, 0, 0] == 0.0


def test_pool_against_torch_max_pool2d():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(31)
    for P, Q in [(2, 2), (7, 6), (6, 9), (13, 13), (3, 2)]:
        y = rng.standard_normal((2, 3, P, Q))
        t = torch.from_numpy(y)
        ref_pool = torch.nn.functional.max_pool2d(t, 2).numpy()
        ref_both = torch.nn.functional.max_pool2d(torch.relu(t), 2).numpy()
        assert np.array_equal(oracle.relu_pool(y, relu=False, pool=True), ref_pool)
        assert np.array_equal(oracle.relu_pool(y, relu=True, pool=True), ref_both)


def test_relu_and_pool_commute():
    # ReLU is monotone, so it commutes with the max: the order the kernels
    # apply them in cannot change the result
    y = np.random.default_rng(32).standard_normal((2, 2, 6, 8))
    relu_then_pool = oracle.relu_pool(y, relu=True, pool=True)
    pool_then_relu = oracle.relu_pool(oracle.relu_pool(y, relu=False, pool=True),
                                      relu=True, pool=False)
    assert np.array_equal(relu_then_pool, pool_then_relu)


def test_pool_maxima_are_maxnum():
    y = np.array([[np.nan, 1.0], [-2.0, 0.5]]).reshape(1, 1, 2, 2)
    assert oracle.relu_pool(y, relu=False, pool=True)[0, 0, 0, 0] == 1.0
    assert np.isnan(oracle.relu_pool(np.full((1, 1, 2, 2), np.nan), False, True)).all()
    assert oracle.relu_pool(np.array([np.nan]).reshape(1, 1, 1, 1), True, False)[0, 0, 0, 0] == 0.0


def test_conv_bias_relu_pool_chain():
    # delta filter and bias -8.5 on the ramp: y = X - 8.5; the bias comes
    # before the ReLU, so only the bottom rows survive
    y = oracle.conv2d(ramp16(), np.ones((1, 1, 1, 1)), np.array([-8.5]))
    out = oracle.relu_pool(y, relu=True, pool=True)
    assert np.array_equal(out[0, 0], [[0.0, 0.0], [14.0 - 8.5, 16.0 - 8.5]])


# ---------------------------------------------------------------- input recipe
def test_layer_shapes_and_recipe():
    L = workloads.LAYERS["mid_3x3_fp32"]
    x, w, b = workloads.make_inputs(L)
    assert x.shape == (1, 512, 13, 13) and w.shape == (1024, 512, 3, 3) and b.shape == (1024,)
    assert x.dtype == np.float32 and np.all(np.abs(x) <= 1)
    assert abs(float(w.std()) - np.sqrt(2 / (512 * 9))) < 2e-4
    L = workloads.LAYERS["stem_7x7_s2_bf16"].replace(N=2)
    x, w, b = workloads.make_inputs(L)
    assert x.dtype == np.uint16 and np.all(b == 0)
    xf = workloads.to_f64(x, "bf16")
    assert 0 <= xf.min() and xf.max() <= 1
    # bf16 rounding is nearest-even on the fp32 value
    v = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5], dtype=np.float32)
    assert list(workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(v))) == \
        [1.0, 1.0 + 4 * 2 ** -8, -2.5]

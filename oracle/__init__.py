"""CPU oracle for im2win forward convolution -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and this
package imports nothing from it: the two share only the seeded generators of
``workloads``.

Parts (the C ones live in ``conv_oracle.c``, plain C, fp64):
  O1 ``conv2d`` / ``conv2d_points`` -- the direct seven-loop convolution
     (cross-correlation, zero padding, dilation, bias after the sum), as the
     OpenCL-Benchmarks page's "Setting: normal" kernel defines it and as
     "CS149 L9 ... The direct version: seven nested loops" describes it.
  O2 ``im2win`` -- the window-tensor repack of "Enabling Memory-efficient
     Im2win Convolution ..." §III-B/§III-C (channel-planar) and §III-D
     (channel-innermost, the NHWC variant), as a copy of element bits.
  O3 ``window_conv`` -- a convolution that reads only O2's window tensor.
  O4 ``im2col_conv`` -- numpy: the im2col matrix (one row per sliding window)
     times the filter matrix, per image ("CS149 L9 ... Rewriting as matrix
     multiply: explicit GEMM").
  O5 ``relu_pool`` -- the fused epilogue of the CS149 page's conv ->
     scale/bias -> max-pool chain ("Fusion: keep intermediates out of
     memory"): ReLU, then the max over non-overlapping 2x2 regions.
The diagonalwise identity for depthwise layers ("Diagonalwise
Refactorization ...", abstract) is exercised in the tests through O1.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "conv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

LAYOUT_CHW = 0   # xw[n][c][h][x*R + r]
LAYOUT_HWC = 1   # xw[n][h][(x*R + r)*C + c]


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2 -fopenmp, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = open_library(_LIB)
    return _lib


def open_library(path: str):
    """Open a compiled copy of conv_oracle.c and declare its signatures."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.oracle_out_dims.argtypes = [P, P, P]
    lib.oracle_out_dims.restype = ctypes.c_int
    lib.oracle_conv2d.argtypes = [P, P, P, P, P]
    lib.oracle_conv2d.restype = None
    lib.oracle_conv2d_points.argtypes = [P, P, P, P, P, i64, P]
    lib.oracle_conv2d_points.restype = None
    lib.oracle_win_width.argtypes = [P]
    lib.oracle_win_width.restype = i64
    lib.oracle_row_pitch.argtypes = [i64, i64]
    lib.oracle_row_pitch.restype = i64
    lib.oracle_row_elems.argtypes = [P, ctypes.c_int]
    lib.oracle_row_elems.restype = i64
    lib.oracle_im2win.argtypes = [P, ctypes.c_int, i64, P, P]
    lib.oracle_im2win.restype = None
    lib.oracle_window_conv.argtypes = [P, ctypes.c_int, P, P, P, P]
    lib.oracle_window_conv.restype = None
    lib.oracle_relu_pool.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P]
    lib.oracle_relu_pool.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def _desc(N, C, H, W, K, R, S, stride, pad, dil, groups) -> np.ndarray:
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    dh, dw = _pair(dil)
    return np.array([N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, groups], dtype=np.int64)


def _pair(v):
    return (int(v), int(v)) if np.isscalar(v) else (int(v[0]), int(v[1]))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def out_dims(x_shape, w_shape, stride=1, pad=0, dil=1, groups=1):
    N, C, H, W = x_shape
    K, _, R, S = w_shape
    d = _desc(N, C, H, W, K, R, S, stride, pad, dil, groups)
    P = ctypes.c_int64()
    Q = ctypes.c_int64()
    _load().oracle_out_dims(d.ctypes.data, ctypes.addressof(P), ctypes.addressof(Q))
    return P.value, Q.value


def _check(x, w, b, groups):
    N, C, H, W = x.shape
    K, Cg, R, S = w.shape
    if C % groups or K % groups or Cg != C // groups:
        raise ValueError("inconsistent groups")
    if b is not None and b.shape != (K,):
        raise ValueError("bias shape")


def conv2d(x, w, b=None, stride=1, pad=0, dil=1, groups=1) -> np.ndarray:
    """O1 on fp64 copies of x, w, b; returns y[N][K][P][Q] in fp64."""
    x, w, b = _f64(x), _f64(w), _f64(b)
    _check(x, w, b, groups)
    N, C, H, W = x.shape
    K, _, R, S = w.shape
    d = _desc(N, C, H, W, K, R, S, stride, pad, dil, groups)
    P, Q = out_dims(x.shape, w.shape, stride, pad, dil, groups)
    y = np.zeros((N, K, max(P, 0), max(Q, 0)), dtype=np.float64)
    if P > 0 and Q > 0:
        _load().oracle_conv2d(d.ctypes.data, _ptr(x), _ptr(w), _ptr(b), y.ctypes.data)
    return y


def conv2d_points(x, w, b, idx, stride=1, pad=0, dil=1, groups=1) -> np.ndarray:
    """O1 at the (n, k, h, w) rows of idx (int array of shape [npts, 4])."""
    x, w, b = _f64(x), _f64(w), _f64(b)
    _check(x, w, b, groups)
    N, C, H, W = x.shape
    K, _, R, S = w.shape
    d = _desc(N, C, H, W, K, R, S, stride, pad, dil, groups)
    idx = np.ascontiguousarray(idx, dtype=np.int64).reshape(-1, 4)
    out = np.zeros(idx.shape[0], dtype=np.float64)
    _load().oracle_conv2d_points(d.ctypes.data, _ptr(x), _ptr(w), _ptr(b),
                                 idx.ctypes.data, idx.shape[0], out.ctypes.data)
    return out


def win_width(x_shape, w_shape, stride=1, pad=0, dil=1, groups=1) -> int:
    N, C, H, W = x_shape
    K, _, R, S = w_shape
    d = _desc(N, C, H, W, K, R, S, stride, pad, dil, groups)
    return int(_load().oracle_win_width(d.ctypes.data))


def window_geometry(x_shape, w_shape, layout, elem_bytes, stride=1, pad=0, dil=1):
    """(rows, row_elems, row_pitch) of the window tensor for the whole batch."""
    N, C, H, W = x_shape
    K, _, R, S = w_shape
    d = _desc(N, C, H, W, K, R, S, stride, pad, dil, 1)
    lib = _load()
    P, Q = out_dims(x_shape, w_shape, stride, pad, dil)
    length = int(lib.oracle_row_elems(d.ctypes.data, layout))
    pitch = int(lib.oracle_row_pitch(length, elem_bytes))
    rows = N * C * P if layout == LAYOUT_CHW else N * P
    return rows, length, pitch


def im2win(x: np.ndarray, R, S, stride=1, pad=0, dil=1, layout=LAYOUT_CHW) -> np.ndarray:
    """O2: the window tensor of x (any of float32/float16/uint16(bf16)/float64),
    as an array of x's storage type with shape [rows, pitch]."""
    x = np.ascontiguousarray(x)
    N, C, H, W = x.shape
    eb = x.dtype.itemsize
    d = _desc(N, C, H, W, 1, R, S, stride, pad, dil, 1)
    rows, _, pitch = window_geometry(x.shape, (1, C, R, S), layout, eb, stride, pad, dil)
    out = np.empty((rows, pitch), dtype=x.dtype)
    if rows and pitch:
        _load().oracle_im2win(d.ctypes.data, layout, eb, x.ctypes.data, out.ctypes.data)
    return out


def window_conv(xw64: np.ndarray, x_shape, w, b=None, stride=1, pad=0, dil=1, groups=1,
                layout=LAYOUT_CHW) -> np.ndarray:
    """O3: convolution from an fp64 window tensor made by ``im2win`` on an fp64 x."""
    w, b = _f64(w), _f64(b)
    xw64 = np.ascontiguousarray(xw64, dtype=np.float64)
    N, C, H, W = x_shape
    K, _, R, S = w.shape
    d = _desc(N, C, H, W, K, R, S, stride, pad, dil, groups)
    P, Q = out_dims(x_shape, w.shape, stride, pad, dil, groups)
    y = np.zeros((N, K, P, Q), dtype=np.float64)
    _load().oracle_window_conv(d.ctypes.data, layout, xw64.ctypes.data, _ptr(w), _ptr(b),
                               y.ctypes.data)
    return y


def im2col_conv(x, w, b=None, stride=1, pad=0, dil=1, groups=1) -> np.ndarray:
    """O4: numpy im2col @ filter matrix in fp64, one image at a time.

    The im2col matrix has one row per output position holding that sliding
    window's C/G*R*S inputs; the filter matrix has one column per output
    channel.  Built with numpy's sliding_window_view; shares nothing with O1."""
    x, w = _f64(x), _f64(w)
    b = _f64(b)
    N, C, H, W = x.shape
    K, Cg, R, S = w.shape
    sh, sw = _pair(stride)
    ph, pw = _pair(pad)
    dh, dw = _pair(dil)
    xp = np.pad(x, ((0, 0), (0, 0), (ph, ph), (pw, pw)))
    span_h, span_w = dh * (R - 1) + 1, dw * (S - 1) + 1
    win = np.lib.stride_tricks.sliding_window_view(xp, (span_h, span_w), axis=(2, 3))
    win = win[:, :, ::sh, ::sw, ::dh, ::dw]            # [N, C, P, Q, R, S]
    P, Q = win.shape[2], win.shape[3]
    Kg = K // groups
    y = np.empty((N, K, P, Q), dtype=np.float64)
    for n in range(N):
        for g in range(groups):
            cols = win[n, g * Cg:(g + 1) * Cg]                      # [Cg, P, Q, R, S]
            cols = cols.transpose(1, 2, 0, 3, 4).reshape(P * Q, Cg * R * S)
            fmat = w[g * Kg:(g + 1) * Kg].reshape(Kg, Cg * R * S).T  # [Cg*R*S, Kg]
            y[n, g * Kg:(g + 1) * Kg] = (cols @ fmat).T.reshape(Kg, P, Q)
    if b is not None:
        y += b[None, :, None, None]
    return y


def pooled_dims(P, Q, pool=True):
    """Extent of O5's output: P/2 x Q/2 (floor) with pooling, else P x Q."""
    return (P // 2, Q // 2) if pool else (P, Q)


def relu_pool(y, relu=True, pool=True) -> np.ndarray:
    """O5 on an fp64 copy of the conv output y[N][K][P][Q]."""
    y = _f64(y)
    N, K, P, Q = y.shape
    P2, Q2 = pooled_dims(P, Q, pool)
    out = np.zeros((N, K, P2, Q2), dtype=np.float64)
    if out.size:
        shape = np.array([N, K, P, Q], dtype=np.int64)
        _load().oracle_relu_pool(shape.ctypes.data, int(bool(relu)), int(bool(pool)),
                                 y.ctypes.data, out.ctypes.data)
    return out

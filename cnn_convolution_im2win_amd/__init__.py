"""im2win forward convolution for AMD Instinct MI355X (gfx950).

Python binding of the C ABI in ``include/conv_im2win.h``: the functions here
carry the C entry points' names and only marshal arguments (shapes into a
descriptor, torch tensors into device pointers, the current HIP stream);
every step of the computation runs in the library's HIP kernels.  PyTorch
supplies device memory and streams.

    y = conv2d(x, w, b, stride=1, padding=1)          # F.conv2d-style helper
    y = conv2d(x, w, b, 1, 1, flags=CIW_FLAG_RELU | CIW_FLAG_MAXPOOL2)   # fused epilogue
    y = conv2d(x, w, None, 1, 1, flags=CIW_FLAG_IMPLICIT)  # window rows built in LDS
    y = conv2d_fwd(x, w, b, y, workspace, ...)        # the C entry point
    xw = conv_im2win_transform(x, R, S, ...)          # the repack alone
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple, Union

from . import _lib
from ._lib import (CIW_BF16, CIW_F16, CIW_F32, CIW_FLAG_FP32_MFMA, CIW_FLAG_FP32_VALU,
                   CIW_NOALLOC_SCRATCH_BYTES,
                   CIW_FLAG_GENERIC,
                   CIW_FLAG_IMPLICIT, CIW_FLAG_MAXPOOL2,
                   CIW_FLAG_NO_SPLIT, CIW_FLAG_RELU, CIW_FLAG_WINDOW_READY, CIW_WIN_CHW,
                   CIW_WIN_HWC, ConvDesc, Im2winError, LIB_PATH, status_string)

IntPair = Union[int, Sequence[int]]

__all__ = [
    "conv2d", "conv2d_fwd", "conv2d_fwd_noalloc", "conv2d_dw_fwd", "conv_im2win_transform",
    "conv_im2win_output_dims", "conv2d_output_dims", "conv_im2win_window_geometry",
    "conv_im2win_window_bytes",
    "conv2d_workspace_bytes", "conv2d_implicit_workspace_bytes", "make_desc", "Im2winError", "status_string", "LIB_PATH",
    "CIW_F32", "CIW_F16", "CIW_BF16", "CIW_WIN_CHW", "CIW_WIN_HWC",
    "CIW_FLAG_WINDOW_READY", "CIW_FLAG_NO_SPLIT", "CIW_FLAG_GENERIC", "CIW_FLAG_RELU",
    "CIW_FLAG_MAXPOOL2", "CIW_FLAG_IMPLICIT", "CIW_FLAG_FP32_MFMA", "CIW_FLAG_FP32_VALU",
    "CIW_NOALLOC_SCRATCH_BYTES",
]


def _pair(v: IntPair) -> Tuple[int, int]:
    if isinstance(v, int):
        return v, v
    a, b = v
    return int(a), int(b)


def make_desc(x_shape, w_shape, stride: IntPair = 1, padding: IntPair = 0,
              dilation: IntPair = 1, groups: int = 1) -> ConvDesc:
    N, C, H, W = (int(v) for v in x_shape)
    K, _, R, S = (int(v) for v in w_shape)
    sh, sw = _pair(stride)
    ph, pw = _pair(padding)
    dh, dw = _pair(dilation)
    return ConvDesc(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, int(groups))


def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: CIW_F32, torch.float16: CIW_F16, torch.bfloat16: CIW_BF16}
    if t not in codes:
        raise TypeError(f"unsupported dtype {t}")
    return codes[t]


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _need_device(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


# ------------------------------------------------------------------ queries
def conv_im2win_output_dims(desc: ConvDesc) -> Tuple[int, int]:
    P, Q = ctypes.c_int64(), ctypes.c_int64()
    _lib.check(_lib.load().conv_im2win_output_dims(ctypes.byref(desc), ctypes.byref(P),
                                                   ctypes.byref(Q)), "conv_im2win_output_dims")
    return P.value, Q.value


def conv2d_output_dims(desc: ConvDesc, flags: int = 0) -> Tuple[int, int]:
    """Extent of the output conv2d_fwd writes with these flags (P/2 x Q/2
    with CIW_FLAG_MAXPOOL2)."""
    P, Q = ctypes.c_int64(), ctypes.c_int64()
    _lib.check(_lib.load().conv2d_output_dims(ctypes.byref(desc), int(flags), ctypes.byref(P),
                                              ctypes.byref(Q)), "conv2d_output_dims")
    return P.value, Q.value


def conv_im2win_window_geometry(desc: ConvDesc, dtype: int, layout: int) -> Tuple[int, int, int]:
    rows, elems, pitch = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _lib.check(_lib.load().conv_im2win_window_geometry(
        ctypes.byref(desc), dtype, layout, ctypes.byref(rows), ctypes.byref(elems),
        ctypes.byref(pitch)), "conv_im2win_window_geometry")
    return rows.value, elems.value, pitch.value


def conv_im2win_window_bytes(desc: ConvDesc, dtype: int, layout: int, n_images: int) -> int:
    out = ctypes.c_size_t()
    _lib.check(_lib.load().conv_im2win_window_bytes(ctypes.byref(desc), dtype, layout,
                                                    int(n_images), ctypes.byref(out)),
               "conv_im2win_window_bytes")
    return out.value


def conv2d_workspace_bytes(desc: ConvDesc, in_dtype: int, n_images: int) -> int:
    out = ctypes.c_size_t()
    _lib.check(_lib.load().conv2d_workspace_bytes(ctypes.byref(desc), in_dtype, int(n_images),
                                                  ctypes.byref(out)), "conv2d_workspace_bytes")
    return out.value


def conv2d_implicit_workspace_bytes(desc: ConvDesc, in_dtype: int, out_dtype: int,
                                    flags: int = 0) -> int:
    """Workspace of conv2d_fwd with CIW_FLAG_IMPLICIT (window rows built in
    LDS); raises Im2winError (unsupported) for layers that kernel does not run."""
    out = ctypes.c_size_t()
    _lib.check(_lib.load().conv2d_implicit_workspace_bytes(
        ctypes.byref(desc), in_dtype, out_dtype, int(flags), ctypes.byref(out)),
        "conv2d_implicit_workspace_bytes")
    return out.value


# ------------------------------------------------------------------ calls
def conv_im2win_transform(x, R: int, S: int, stride: IntPair = 1, padding: IntPair = 0,
                          dilation: IntPair = 1, layout: int = CIW_WIN_CHW, out=None,
                          stream=None):
    """Repack x (NCHW) into its window tensor; returns [rows, pitch] of x's dtype."""
    import torch
    _need_device(x)
    if x.dim() != 4:
        raise ValueError("x must be 4-D")
    desc = make_desc(x.shape, (1, x.shape[1], R, S), stride, padding, dilation, 1)
    dt = _dtype_code(x.dtype)
    rows, _, pitch = conv_im2win_window_geometry(desc, dt, layout)
    if out is None:
        out = torch.empty((x.shape[0] * rows, pitch), dtype=x.dtype, device=x.device)
    _need_device(out)
    if out.numel() * out.element_size() < x.shape[0] * rows * pitch * x.element_size():
        raise ValueError("out is smaller than the window tensor")
    _lib.check(_lib.load().conv_im2win_transform(ctypes.byref(desc), dt, layout, _ptr(x),
                                                 _ptr(out), _stream(stream)),
               "conv_im2win_transform")
    return out


def _check_shapes(desc: ConvDesc, x, w, bias, y, flags: int = 0) -> None:
    """Host-side shape and dtype checks: the C ABI takes every extent from the
    descriptor, so a tensor that disagrees with it must never reach a kernel."""
    import torch
    if x is not None and (x.dim() != 4 or tuple(x.shape) != (desc.N, desc.C, desc.H, desc.W)):
        raise ValueError(f"x shape {tuple(x.shape)} does not match the descriptor")
    if w.dim() != 4 or tuple(w.shape) != (desc.K, desc.C // max(desc.groups, 1), desc.R, desc.S):
        raise ValueError(f"weight shape {tuple(w.shape)} does not match C/groups = "
                         f"{desc.C}/{desc.groups}")
    if x is not None and x.dtype != w.dtype:
        raise ValueError("x and weight must share a dtype")
    if bias is not None and (bias.dim() != 1 or bias.numel() != desc.K or bias.dtype != w.dtype):
        raise ValueError("bias must be a [K] tensor of the weight's dtype")
    P, Q = conv2d_output_dims(desc, flags)
    if tuple(y.shape) != (desc.N, desc.K, P, Q):
        raise ValueError(f"y shape {tuple(y.shape)} != {(desc.N, desc.K, P, Q)}")
    if y.dtype not in (w.dtype, torch.float32):
        raise ValueError("y dtype must be the input dtype or float32")


def _conv_call(fn_name, x, w, bias, y, workspace, stride, padding, dilation, groups, flags,
               stream, x_shape=None):
    shape = x.shape if x is not None else x_shape
    desc = make_desc(shape, w.shape, stride, padding, dilation, groups)
    _need_device(x, w, bias, y, workspace)
    _check_shapes(desc, x, w, bias, y, flags)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = getattr(_lib.load(), fn_name)(
        ctypes.byref(desc), _dtype_code(w.dtype), _dtype_code(y.dtype), _ptr(x), _ptr(w),
        _ptr(bias), _ptr(y), _ptr(workspace), ws_bytes, int(flags), _stream(stream))
    _lib.check(st, fn_name)
    return y


def conv2d_fwd(x, w, bias, y, workspace, stride: IntPair = 1, padding: IntPair = 0,
               dilation: IntPair = 1, flags: int = 0, stream=None, x_shape=None):
    """Dense (groups = 1) im2win convolution into the preallocated y.
    x may be None with CIW_FLAG_WINDOW_READY (then pass x_shape)."""
    return _conv_call("conv2d_fwd", x, w, bias, y, workspace, stride, padding, dilation, 1,
                      flags, stream, x_shape)


def conv2d_fwd_noalloc(x, w, bias, y, stride: IntPair = 1, padding: IntPair = 0,
                       dilation: IntPair = 1, flags: int = 0, stream=None):
    """Dense (groups = 1) im2win convolution into the preallocated y with no
    workspace argument: the library's own device array
    (CIW_NOALLOC_SCRATCH_BYTES per GPU) serves as the workspace, so nothing
    is allocated on this path.  Calls that overlap on one GPU race on it."""
    desc = make_desc(x.shape, w.shape, stride, padding, dilation, 1)
    _need_device(x, w, bias, y)
    _check_shapes(desc, x, w, bias, y, flags)
    st = _lib.load().conv2d_fwd_noalloc(
        ctypes.byref(desc), _dtype_code(w.dtype), _dtype_code(y.dtype), _ptr(x), _ptr(w),
        _ptr(bias), _ptr(y), int(flags), _stream(stream))
    _lib.check(st, "conv2d_fwd_noalloc")
    return y


def conv2d_dw_fwd(x, w, bias, y, workspace, stride: IntPair = 1, padding: IntPair = 0,
                  dilation: IntPair = 1, flags: int = 0, stream=None, x_shape=None):
    """Depthwise (groups = C = K) im2win convolution into the preallocated y."""
    shape = x.shape if x is not None else x_shape
    return _conv_call("conv2d_dw_fwd", x, w, bias, y, workspace, stride, padding, dilation,
                      int(shape[1]), flags, stream, x_shape)


def conv2d(x, weight, bias=None, stride: IntPair = 1, padding: IntPair = 0,
           dilation: IntPair = 1, groups: int = 1, out_dtype=None, workspace=None,
           flags: int = 0, stream=None):
    """F.conv2d-style helper: allocates y (and a full-batch workspace unless one
    is given) with torch, then calls conv2d_fwd or conv2d_dw_fwd."""
    import torch
    _need_device(x, weight, bias)
    if x.dim() != 4 or weight.dim() != 4:
        raise ValueError("x and weight must be 4-D")
    desc = make_desc(x.shape, weight.shape, stride, padding, dilation, groups)
    P, Q = conv2d_output_dims(desc, flags)
    out_dtype = x.dtype if out_dtype is None else out_dtype
    y = torch.empty((x.shape[0], weight.shape[0], P, Q), dtype=out_dtype, device=x.device)
    depthwise = groups > 1
    if workspace is None and flags & CIW_FLAG_IMPLICIT:
        nbytes = conv2d_implicit_workspace_bytes(desc, _dtype_code(x.dtype), _dtype_code(out_dtype),
                                                 flags)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=x.device)
    elif workspace is None:
        nbytes = conv2d_workspace_bytes(desc, _dtype_code(x.dtype), max(int(x.shape[0]), 1))
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=x.device)
    fn = conv2d_dw_fwd if depthwise else conv2d_fwd
    return fn(x, weight, bias, y, workspace, stride, padding, dilation, flags, stream)

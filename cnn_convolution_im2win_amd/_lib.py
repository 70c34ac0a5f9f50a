"""ctypes view of the C ABI in include/conv_im2win.h (no logic of its own).

The shared library is ``libconv_im2win.so`` next to this file, built by
``cnn_convolution_im2win_amd.build``.  There is no fallback: if it is
missing, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libconv_im2win.so")

CIW_OK = 0
CIW_ERR_INVALID_ARG = -1
CIW_ERR_UNSUPPORTED = -2
CIW_ERR_WORKSPACE = -3
CIW_ERR_HIP = -4

CIW_F32, CIW_F16, CIW_BF16 = 0, 1, 2
CIW_WIN_CHW, CIW_WIN_HWC = 0, 1

CIW_FLAG_WINDOW_READY = 0x1
CIW_FLAG_NO_SPLIT = 0x2
CIW_FLAG_GENERIC = 0x4
CIW_FLAG_RELU = 0x8
CIW_FLAG_MAXPOOL2 = 0x10
CIW_FLAG_IMPLICIT = 0x20
CIW_FLAG_FP32_MFMA = 0x40
CIW_FLAG_FP32_VALU = 0x80

# the exported entry points, in header order
ENTRY_POINTS = (
    "conv_im2win_output_dims",
    "conv2d_output_dims",
    "conv_im2win_window_geometry",
    "conv_im2win_window_bytes",
    "conv_im2win_transform",
    "conv2d_workspace_bytes",
    "conv2d_implicit_workspace_bytes",
    "conv2d_fwd",
    "conv2d_fwd_noalloc",
    "conv2d_dw_fwd",
    "conv_im2win_status_string",
)

# bytes of the device array conv2d_fwd_noalloc uses as its workspace
CIW_NOALLOC_SCRATCH_BYTES = 32 << 20


class ConvDesc(ctypes.Structure):
    """Mirror of ciw_conv_desc."""
    _fields_ = [
        ("N", ctypes.c_int64), ("C", ctypes.c_int64), ("H", ctypes.c_int64),
        ("W", ctypes.c_int64), ("K", ctypes.c_int64), ("R", ctypes.c_int64),
        ("S", ctypes.c_int64),
        ("stride_h", ctypes.c_int32), ("stride_w", ctypes.c_int32),
        ("pad_h", ctypes.c_int32), ("pad_w", ctypes.c_int32),
        ("dil_h", ctypes.c_int32), ("dil_w", ctypes.c_int32),
        ("groups", ctypes.c_int32),
    ]


class Im2winError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def open_library(path: str):
    """Open a build of the library at `path` with the ctypes signatures of
    the C ABI set (the package's own library, or an ablation variant built
    by ``build.build_variants``)."""
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m cnn_convolution_im2win_amd.build` "
            "(or __graft_entry__.build()); there is no CPU fallback")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    D = ctypes.POINTER(ConvDesc)
    i32, u32, i64 = ctypes.c_int32, ctypes.c_uint32, ctypes.c_int64
    pi64 = ctypes.POINTER(ctypes.c_int64)
    psz = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "conv_im2win_output_dims": [D, pi64, pi64],
        "conv2d_output_dims": [D, u32, pi64, pi64],
        "conv_im2win_window_geometry": [D, i32, i32, pi64, pi64, pi64],
        "conv_im2win_window_bytes": [D, i32, i32, i64, psz],
        "conv_im2win_transform": [D, i32, i32, P, P, P],
        "conv2d_workspace_bytes": [D, i32, i64, psz],
        "conv2d_implicit_workspace_bytes": [D, i32, i32, u32, psz],
        "conv2d_fwd": [D, i32, i32, P, P, P, P, P, ctypes.c_size_t, u32, P],
        "conv2d_fwd_noalloc": [D, i32, i32, P, P, P, P, u32, P],
        "conv2d_dw_fwd": [D, i32, i32, P, P, P, P, P, ctypes.c_size_t, u32, P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.conv_im2win_status_string.argtypes = [ctypes.c_int]
    lib.conv_im2win_status_string.restype = ctypes.c_char_p
    return lib


def load():
    """Open the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = open_library(LIB_PATH)
    return _lib


def status_string(status: int) -> str:
    return load().conv_im2win_status_string(int(status)).decode()


def check(status: int, where: str) -> None:
    if status != CIW_OK:
        raise Im2winError(status, where)

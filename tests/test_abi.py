"""C-ABI checks that need no GPU: the library loads, exports every entry point
the header declares, its shape arithmetic agrees with the oracle's, and every
invalid call is rejected before anything is launched (these calls never get
far enough to touch a pointer, so fake addresses are safe here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "conv_im2win.h")

m = pytest.importorskip("cnn_convolution_im2win_amd")
from cnn_convolution_im2win_amd import _lib  # noqa: E402


def lib():
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^(?:ciw_status|const char\*)\s+(\w+)\s*\(", text, flags=re.M)


def test_header_and_binding_agree():
    names = declared_functions()
    assert len(names) == 11
    assert tuple(names) == _lib.ENTRY_POINTS


def test_library_exports_every_declared_symbol():
    L = lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    assert m.status_string(0) == "success"
    for s in (-1, -2, -3, -4):
        assert m.status_string(s) and m.status_string(s) != "unknown status"
    assert m.status_string(-99) == "unknown status"


def desc_of(L: workloads.Layer):
    return m.make_desc(L.x_shape, L.w_shape, L.stride, L.pad, L.dil, L.groups)


def test_output_dims_match_oracle():
    rng = np.random.default_rng(0)
    layers = list(workloads.LAYERS.values()) + [workloads.random_layer(rng) for _ in range(50)]
    for L in layers:
        assert m.conv_im2win_output_dims(desc_of(L)) == oracle.out_dims(
            L.x_shape, L.w_shape, L.stride, L.pad, L.dil), L


def test_window_geometry_matches_oracle():
    rng = np.random.default_rng(1)
    layers = list(workloads.LAYERS.values()) + [workloads.random_layer(rng) for _ in range(50)]
    for L in layers:
        d = desc_of(L)
        for code, eb in ((m.CIW_F32, 4), (m.CIW_F16, 2), (m.CIW_BF16, 2)):
            for lay in (m.CIW_WIN_CHW, m.CIW_WIN_HWC):
                rows, elems, pitch = m.conv_im2win_window_geometry(d, code, lay)
                o_rows, o_len, o_pitch = oracle.window_geometry(
                    L.x_shape, L.w_shape, lay, eb, L.stride, L.pad, L.dil)
                assert (rows * L.N, elems, pitch) == (o_rows, o_len, o_pitch), L
                assert m.conv_im2win_window_bytes(d, code, lay, L.N) == o_rows * o_pitch * eb


def test_window_sizes_of_the_five_layers():
    # window tensor bytes of the five layers (CHW for fp32 and depthwise,
    # HWC for fp16/bf16): 0.213, 1.278, 159.65, 138.08 and 176.16 MB
    want = {"tiny_3x3_fp32": 212992, "mid_3x3_fp32": 1277952, "resnet_3x3_fp16": 159645696,
            "stem_7x7_s2_bf16": 138084352, "dw_3x3_fp32": 176160768}
    for name, L in workloads.LAYERS.items():
        code = {"f32": m.CIW_F32, "f16": m.CIW_F16, "bf16": m.CIW_BF16}[L.dtype]
        lay = m.CIW_WIN_CHW if L.dtype == "f32" else m.CIW_WIN_HWC
        assert m.conv_im2win_window_bytes(desc_of(L), code, lay, L.N) == want[name]


def test_workspace_covers_window():
    for L in workloads.LAYERS.values():
        code = {"f32": m.CIW_F32, "f16": m.CIW_F16, "bf16": m.CIW_BF16}[L.dtype]
        lay = m.CIW_WIN_CHW if L.dtype == "f32" else m.CIW_WIN_HWC
        d = desc_of(L)
        assert m.conv2d_workspace_bytes(d, code, L.N) >= m.conv_im2win_window_bytes(d, code, lay, L.N)
        assert m.conv2d_workspace_bytes(d, code, 1) >= m.conv_im2win_window_bytes(d, code, lay, 1)


# ------------------------------------------------------------------ validation
FAKE = 0x1000_0000          # 16-byte aligned, never dereferenced by these calls


def call_fwd(d, in_dt=0, out_dt=0, x=FAKE, w=FAKE, b=None, y=FAKE, ws=FAKE, ws_bytes=0,
             flags=0, fn="conv2d_fwd"):
    return getattr(lib(), fn)(ctypes.byref(d) if d is not None else None, in_dt, out_dt, x, w,
                              b, y, ws, ws_bytes, flags, None)


def valid_desc(**kw):
    base = dict(N=2, C=4, H=8, W=8, K=6, R=3, S=3, stride_h=1, stride_w=1, pad_h=1, pad_w=1,
                dil_h=1, dil_w=1, groups=1)
    base.update(kw)
    return _lib.ConvDesc(**base)


@pytest.mark.parametrize("field,value", [
    ("C", 0), ("H", 0), ("W", -1), ("K", 0), ("R", 0), ("S", 0), ("N", -1),
    ("stride_h", 0), ("stride_w", -2), ("pad_h", -1), ("dil_w", 0), ("groups", 0),
    ("groups", 3), ("R", 20),   # groups must divide C and K; window larger than padded input
])
def test_invalid_descriptor(field, value):
    d = valid_desc(**{field: value})
    assert call_fwd(d) == _lib.CIW_ERR_INVALID_ARG
    P, Q = ctypes.c_int64(), ctypes.c_int64()
    assert lib().conv_im2win_output_dims(ctypes.byref(d), ctypes.byref(P), ctypes.byref(Q)) == \
        _lib.CIW_ERR_INVALID_ARG


def test_null_descriptor_and_outputs():
    assert call_fwd(None) == _lib.CIW_ERR_INVALID_ARG
    d = valid_desc()
    assert lib().conv_im2win_window_bytes(ctypes.byref(d), 0, 0, 1, None) == _lib.CIW_ERR_INVALID_ARG
    assert lib().conv2d_workspace_bytes(ctypes.byref(d), 0, 0, None) == _lib.CIW_ERR_INVALID_ARG


def test_unsupported_groups():
    assert call_fwd(valid_desc(C=4, K=4, groups=2)) == _lib.CIW_ERR_UNSUPPORTED
    # depthwise entry point wants groups == C == K
    assert call_fwd(valid_desc(C=4, K=8, groups=4), fn="conv2d_dw_fwd") == _lib.CIW_ERR_UNSUPPORTED
    assert call_fwd(valid_desc(C=4, K=4, groups=1), fn="conv2d_dw_fwd") == _lib.CIW_ERR_INVALID_ARG
    assert call_fwd(valid_desc(C=4, K=4, groups=4)) == _lib.CIW_ERR_UNSUPPORTED


@pytest.mark.parametrize("in_dt,out_dt", [(0, 1), (0, 2), (1, 2), (2, 1), (3, 0), (0, 7)])
def test_bad_dtype_pairs(in_dt, out_dt):
    assert call_fwd(valid_desc(), in_dt, out_dt) == _lib.CIW_ERR_INVALID_ARG


@pytest.mark.parametrize("which", ["x", "w", "y", "ws"])
def test_null_and_misaligned_pointers(which):
    kw = {which: None}
    assert call_fwd(valid_desc(), ws_bytes=1 << 30, **kw) == _lib.CIW_ERR_INVALID_ARG
    kw = {which: FAKE + 4}
    assert call_fwd(valid_desc(), ws_bytes=1 << 30, **kw) == _lib.CIW_ERR_INVALID_ARG


def test_misaligned_bias():
    assert call_fwd(valid_desc(), b=FAKE + 2, ws_bytes=1 << 30) == _lib.CIW_ERR_INVALID_ARG
    assert call_fwd(valid_desc(), 1, 1, b=FAKE + 1, ws_bytes=1 << 30) == _lib.CIW_ERR_INVALID_ARG


def test_unknown_flags():
    assert call_fwd(valid_desc(), ws_bytes=1 << 30, flags=0x100) == _lib.CIW_ERR_INVALID_ARG
    both = _lib.CIW_FLAG_FP32_MFMA | _lib.CIW_FLAG_FP32_VALU
    assert call_fwd(valid_desc(), ws_bytes=1 << 30, flags=both) == _lib.CIW_ERR_INVALID_ARG


def test_implicit_flag_host_checks():
    # fp32 in LDS has no pooled form and runs only 3x3 and 1x1 filters (both
    # refused before any launch); the flag combinations it forbids
    pooled = _lib.CIW_FLAG_IMPLICIT | _lib.CIW_FLAG_MAXPOOL2
    assert call_fwd(valid_desc(), ws_bytes=1 << 30, flags=pooled) == _lib.CIW_ERR_UNSUPPORTED
    assert call_fwd(valid_desc(R=5, S=5, pad_h=2, pad_w=2), ws_bytes=1 << 30,
                    flags=_lib.CIW_FLAG_IMPLICIT) == _lib.CIW_ERR_UNSUPPORTED
    both = _lib.CIW_FLAG_IMPLICIT | _lib.CIW_FLAG_WINDOW_READY
    assert call_fwd(valid_desc(), ws_bytes=1 << 30, flags=both) == _lib.CIW_ERR_INVALID_ARG


def test_pooled_output_dims_match_oracle():
    rng = np.random.default_rng(1)
    layers = list(workloads.LAYERS.values()) + [workloads.random_layer(rng) for _ in range(50)]
    for L in layers:
        P, Q = oracle.out_dims(L.x_shape, L.w_shape, L.stride, L.pad, L.dil)
        d = desc_of(L)
        assert m.conv2d_output_dims(d) == (P, Q)
        assert m.conv2d_output_dims(d, m.CIW_FLAG_RELU) == (P, Q)
        if P >= 2 and Q >= 2:
            assert m.conv2d_output_dims(d, m.CIW_FLAG_MAXPOOL2) == oracle.pooled_dims(P, Q), L


@pytest.mark.parametrize("H,W", [(1, 8), (8, 1), (1, 1)])
def test_pool_needs_a_2x2_region(H, W):
    # 1x1 filter, no padding: P = H, Q = W; a 1-wide output has no 2x2 region
    d = valid_desc(H=H, W=W, R=1, S=1, pad_h=0, pad_w=0)
    P, Q = ctypes.c_int64(), ctypes.c_int64()
    assert lib().conv2d_output_dims(ctypes.byref(d), m.CIW_FLAG_MAXPOOL2, ctypes.byref(P),
                                    ctypes.byref(Q)) == _lib.CIW_ERR_INVALID_ARG
    for fn in ("conv2d_fwd", "conv2d_dw_fwd"):
        dd = d if fn == "conv2d_fwd" else valid_desc(H=H, W=W, R=1, S=1, pad_h=0, pad_w=0,
                                                      C=4, K=4, groups=4)
        assert call_fwd(dd, ws_bytes=1 << 30, flags=m.CIW_FLAG_MAXPOOL2, fn=fn) == \
            _lib.CIW_ERR_INVALID_ARG
        assert call_fwd(dd, ws_bytes=1 << 30, flags=m.CIW_FLAG_MAXPOOL2 | m.CIW_FLAG_RELU,
                        fn=fn) == _lib.CIW_ERR_INVALID_ARG


def test_workspace_too_small():
    d = valid_desc()
    one = m.conv2d_workspace_bytes(d, 0, 1)
    assert call_fwd(d, ws_bytes=one - 1) == _lib.CIW_ERR_WORKSPACE
    assert call_fwd(d, ws_bytes=0) == _lib.CIW_ERR_WORKSPACE
    # a window-ready call needs the full-batch window tensor
    full = m.conv2d_workspace_bytes(d, 0, 2)
    assert call_fwd(d, x=None, ws_bytes=full - 16, flags=m.CIW_FLAG_WINDOW_READY) == \
        _lib.CIW_ERR_WORKSPACE


def test_int32_overflow_is_unsupported():
    d = valid_desc(N=1 << 16, C=1 << 10, H=64, W=64)
    assert call_fwd(d) == _lib.CIW_ERR_UNSUPPORTED


@pytest.mark.parametrize("fields", [
    # 2^20 * 2^20 * 2^20 * 16 = 2^64: wraps to 0 in an unchecked int64 product
    dict(N=1 << 20, C=1 << 20, H=1 << 20, W=16, K=1 << 20, R=1, S=1, pad_h=0, pad_w=0),
    # 2^21 * 2^21 * 2^21 * 2^1 = 2^64 through the output tensor
    dict(N=1 << 21, C=1, H=1 << 21, W=2, K=1 << 21, R=1, S=1, pad_h=0, pad_w=0),
    # filter tensor K * C * R * S = 2^31 * ... past int64
    dict(N=1, C=1 << 30, H=1, W=1, K=(1 << 31) - 1, R=1, S=1, pad_h=0, pad_w=0),
    # window row length: Wwin * R * C with a huge dilation
    dict(N=1, C=1 << 16, H=8, W=8, K=1, R=3, S=1 << 16, pad_h=1, pad_w=1 << 30, dil_w=1 << 14),
    # largest legal extents in every field
    dict(N=(1 << 31) - 1, C=(1 << 31) - 1, H=(1 << 31) - 1, W=(1 << 31) - 1, K=(1 << 31) - 1,
         R=1, S=1, pad_h=0, pad_w=0),
])
def test_wrapping_descriptors_are_unsupported(fields):
    """Extents whose products wrap a 64-bit integer must be rejected, not
    accepted with a wrapped size (the host checks every partial product)."""
    d = valid_desc(**fields)
    assert call_fwd(d) == _lib.CIW_ERR_UNSUPPORTED
    P, Q = ctypes.c_int64(), ctypes.c_int64()
    assert lib().conv_im2win_output_dims(ctypes.byref(d), ctypes.byref(P), ctypes.byref(Q)) == \
        _lib.CIW_ERR_UNSUPPORTED
    out = ctypes.c_size_t()
    for lay in (m.CIW_WIN_CHW, m.CIW_WIN_HWC):
        assert lib().conv_im2win_window_bytes(ctypes.byref(d), 0, lay, 1, ctypes.byref(out)) == \
            _lib.CIW_ERR_UNSUPPORTED
    assert lib().conv2d_workspace_bytes(ctypes.byref(d), 0, 1, ctypes.byref(out)) == \
        _lib.CIW_ERR_UNSUPPORTED


def test_window_bytes_of_huge_image_counts_do_not_wrap():
    d = valid_desc()
    out = ctypes.c_size_t()
    assert lib().conv_im2win_window_bytes(ctypes.byref(d), 0, 0, 1 << 62, ctypes.byref(out)) == \
        _lib.CIW_ERR_UNSUPPORTED
    # a workspace query for more images than the batch is the full-batch size
    assert lib().conv2d_workspace_bytes(ctypes.byref(d), 0, 1 << 62, ctypes.byref(out)) == _lib.CIW_OK
    assert out.value == m.conv2d_workspace_bytes(d, 0, d.N)


def test_empty_batch_is_a_no_op():
    d = valid_desc(N=0)
    assert call_fwd(d, x=None, w=None, y=None, ws=None) == _lib.CIW_OK
    assert lib().conv_im2win_transform(ctypes.byref(d), 0, 0, None, None, None) == _lib.CIW_OK


def test_transform_validation():
    d = valid_desc()
    L = lib()
    assert L.conv_im2win_transform(ctypes.byref(d), 0, 2, FAKE, FAKE, None) == _lib.CIW_ERR_INVALID_ARG
    assert L.conv_im2win_transform(ctypes.byref(d), 0, 0, None, FAKE, None) == _lib.CIW_ERR_INVALID_ARG
    assert L.conv_im2win_transform(ctypes.byref(d), 0, 0, FAKE, FAKE + 8, None) == _lib.CIW_ERR_INVALID_ARG
    assert L.conv_im2win_transform(ctypes.byref(d), 5, 0, FAKE, FAKE, None) == _lib.CIW_ERR_INVALID_ARG


# ---------------------------------------------------------- allocation-free entry point
def call_noalloc(d, in_dt=0, out_dt=0, x=FAKE, w=FAKE, b=None, y=FAKE, flags=0):
    return lib().conv2d_fwd_noalloc(ctypes.byref(d) if d is not None else None, in_dt, out_dt,
                                    x, w, b, y, flags, None)


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    assert re.search(r"#define CIW_NOALLOC_SCRATCH_BYTES \(32u << 20\)", text)
    assert _lib.CIW_NOALLOC_SCRATCH_BYTES == 32 << 20


def test_noalloc_validation_before_any_launch():
    """Every rejection happens before the library touches the runtime (these
    run without a GPU)."""
    assert call_noalloc(None) == _lib.CIW_ERR_INVALID_ARG
    d = valid_desc()
    # a prepared window tensor cannot live in the library's array
    assert call_noalloc(d, x=None, flags=m.CIW_FLAG_WINDOW_READY) == _lib.CIW_ERR_INVALID_ARG
    assert call_noalloc(d, x=None) == _lib.CIW_ERR_INVALID_ARG
    assert call_noalloc(d, y=FAKE + 8) == _lib.CIW_ERR_INVALID_ARG
    assert call_noalloc(d, flags=0x10000) == _lib.CIW_ERR_INVALID_ARG
    assert call_noalloc(d, in_dt=0, out_dt=1) == _lib.CIW_ERR_INVALID_ARG
    assert call_noalloc(valid_desc(C=4, K=4, groups=4)) == _lib.CIW_ERR_UNSUPPORTED
    # one image's window tensor larger than the array: 224 x (226*3*512) x 2 B
    big = valid_desc(N=2, C=512, H=224, W=224, K=64)
    assert m.conv2d_workspace_bytes(big, 1, 1) > _lib.CIW_NOALLOC_SCRATCH_BYTES
    assert call_noalloc(big, in_dt=1, out_dt=1) == _lib.CIW_ERR_WORKSPACE
    assert call_noalloc(valid_desc(N=0), x=None, w=None, y=None) == _lib.CIW_OK

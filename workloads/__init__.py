"""Seeded synthetic convolution layers and dtype codecs.

This module is shared by the CPU oracle (``oracle/``) and by the GPU path
(``cnn_convolution_im2win_amd``) and holds none of the method's arithmetic:
only layer shapes, random draws and bit-level conversions between numpy
arrays and the three element types (fp32, fp16, bf16).

Recipe (every layer): ``numpy.random.default_rng(seed)`` (PCG64) draws, in
fp64 and in this order, the input x, the filters w and the bias b; each is
then rounded to nearest-even into the layer's element type.  bf16 has no
numpy type, so bf16 tensors are carried as ``uint16`` bit patterns.

Layer table.  The im2win paper ("Enabling Memory-efficient Im2win
Convolution with Multi-precision Support on GPU CUDA and Tensor Cores",
§IV-B) benchmarks twelve layers whose table did not survive in the text we
have, so these five synthetic layers stand in for them; "mid_3x3_fp32" is the
exact layer of the OpenCL-Benchmarks page ("Convolution Ops Analysis":
1x512x13x13 input, 1024x512x3x3 weights, stride 1, padding 1, bias).
He-normal means N(0, 2 / fan_in) with fan_in = (C / groups) * R * S.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np

DTYPES = ("f32", "f16", "bf16")
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


@dataclasses.dataclass(frozen=True)
class Layer:
    name: str
    N: int
    C: int
    H: int
    W: int
    K: int
    R: int
    S: int
    stride: Tuple[int, int] = (1, 1)
    pad: Tuple[int, int] = (0, 0)
    dil: Tuple[int, int] = (1, 1)
    groups: int = 1
    dtype: str = "f32"          # input / filter / bias element type
    out_dtype: str = "f32"      # output element type
    x_dist: Tuple = ("uniform", -1.0, 1.0)
    w_dist: Tuple = ("he_normal",)
    b_dist: Optional[Tuple] = ("uniform", -0.1, 0.1)   # None: no bias tensor
    seed: int = 0

    @property
    def x_shape(self):
        return (self.N, self.C, self.H, self.W)

    @property
    def w_shape(self):
        return (self.K, self.C // self.groups, self.R, self.S)

    @property
    def fan_in(self):
        return (self.C // self.groups) * self.R * self.S

    def replace(self, **kw) -> "Layer":
        return dataclasses.replace(self, **kw)


# The five layers, in the order they are listed for this path (index 0..4).
LAYERS: Dict[str, Layer] = {
    "tiny_3x3_fp32": Layer(
        "tiny_3x3_fp32", N=1, C=16, H=32, W=32, K=32, R=3, S=3,
        stride=(1, 1), pad=(1, 1), dtype="f32", out_dtype="f32",
        x_dist=("uniform", -1.0, 1.0), w_dist=("uniform", -0.1, 0.1),
        b_dist=("uniform", -0.1, 0.1), seed=0),
    "mid_3x3_fp32": Layer(
        "mid_3x3_fp32", N=1, C=512, H=13, W=13, K=1024, R=3, S=3,
        stride=(1, 1), pad=(1, 1), dtype="f32", out_dtype="f32",
        x_dist=("uniform", -1.0, 1.0), w_dist=("he_normal",),
        b_dist=("uniform", -0.1, 0.1), seed=1),
    "resnet_3x3_fp16": Layer(
        "resnet_3x3_fp16", N=128, C=64, H=56, W=56, K=64, R=3, S=3,
        stride=(1, 1), pad=(1, 1), dtype="f16", out_dtype="f16",
        x_dist=("normal", 0.0, 1.0), w_dist=("he_normal",),
        b_dist=None, seed=2),
    "stem_7x7_s2_bf16": Layer(
        "stem_7x7_s2_bf16", N=128, C=3, H=224, W=224, K=64, R=7, S=7,
        stride=(2, 2), pad=(3, 3), dtype="bf16", out_dtype="bf16",
        x_dist=("uniform", 0.0, 1.0), w_dist=("he_normal",),
        b_dist=("zeros",), seed=3),
    "dw_3x3_fp32": Layer(
        "dw_3x3_fp32", N=128, C=512, H=14, W=14, K=512, R=3, S=3,
        stride=(1, 1), pad=(1, 1), groups=512, dtype="f32", out_dtype="f32",
        x_dist=("normal", 0.0, 1.0), w_dist=("he_normal",),
        b_dist=("uniform", -0.1, 0.1), seed=4),
}
LAYER_ORDER = list(LAYERS)


# ---------------------------------------------------------------- dtype codecs
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to nearest-even bf16; returns uint16 bit patterns.
    (Inputs here are finite; NaN handling is not needed.)"""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def from_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to the element type (RNE).  bf16 goes through fp32
    first; the result is whatever bf16 value that gives, and that value is the
    input both sides see."""
    if dtype == "f32":
        return a.astype(np.float32)
    if dtype == "f16":
        return a.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(a.astype(np.float32))
    raise ValueError(dtype)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of an element-type array to fp64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a).astype(np.float64)


def storage_dtype(dtype: str):
    return {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]


# ---------------------------------------------------------------- generators
def _draw(rng: np.random.Generator, dist: Tuple, shape, fan_in: int) -> np.ndarray:
    kind = dist[0]
    if kind == "uniform":
        return rng.uniform(dist[1], dist[2], size=shape)
    if kind == "normal":
        return rng.normal(dist[1], dist[2], size=shape)
    if kind == "he_normal":
        return rng.normal(0.0, math.sqrt(2.0 / fan_in), size=shape)
    if kind == "zeros":
        return np.zeros(shape, dtype=np.float64)
    raise ValueError(dist)


def make_inputs(layer: Layer, seed: Optional[int] = None):
    """Seeded host tensors (x, w, b) in the layer's element type; b may be None."""
    rng = np.random.default_rng(layer.seed if seed is None else seed)
    x = _draw(rng, layer.x_dist, layer.x_shape, layer.fan_in)
    w = _draw(rng, layer.w_dist, layer.w_shape, layer.fan_in)
    b = None
    if layer.b_dist is not None:
        b = _draw(rng, layer.b_dist, (layer.K,), layer.fan_in)
    cast = lambda a: None if a is None else from_f64(a, layer.dtype)
    return cast(x), cast(w), cast(b)


def random_layer(rng: np.random.Generator, dtype: str = "f32", depthwise: bool = False,
                 max_hw: int = 12, max_c: int = 12, max_k: int = 12) -> Layer:
    """A small random layer for sweeps (ragged sizes, odd strides/pads/dilations)."""
    while True:
        R = int(rng.choice([1, 2, 3, 5, 7]))
        S = int(rng.choice([1, 2, 3, 5, 7]))
        sh, sw = (int(v) for v in rng.integers(1, 4, size=2))
        ph, pw = (int(v) for v in rng.integers(0, 4, size=2))
        dh, dw = (int(v) for v in rng.integers(1, 3, size=2))
        H = int(rng.integers(1, max_hw + 1))
        W = int(rng.integers(1, max_hw + 1))
        C = int(rng.integers(1, max_c + 1))
        K = C if depthwise else int(rng.integers(1, max_k + 1))
        N = int(rng.integers(1, 4))
        # the window must fit the padded input at least once in each direction
        if H + 2 * ph < dh * (R - 1) + 1 or W + 2 * pw < dw * (S - 1) + 1:
            continue
        out = {"f32": "f32", "f16": "f16", "bf16": "bf16"}[dtype]
        return Layer("random", N=N, C=C, H=H, W=W, K=K, R=R, S=S, stride=(sh, sw),
                     pad=(ph, pw), dil=(dh, dw), groups=C if depthwise else 1,
                     dtype=dtype, out_dtype=out, x_dist=("uniform", -1.0, 1.0),
                     w_dist=("uniform", -0.5, 0.5),
                     b_dist=("uniform", -0.1, 0.1) if rng.integers(0, 2) else None,
                     seed=int(rng.integers(0, 2**31)))

"""Helpers for the GPU tests: host arrays <-> device tensors, tolerances."""
import numpy as np

import workloads

TOL = {"f32": 1e-4, "f16": 2e-2, "bf16": 2e-2}   # max|err| <= TOL * max|ref|


def torch_dtype(name):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[name]


def to_dev(a, dtype: str):
    """Host array of the element type (bf16 as uint16 bits) -> device tensor."""
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to("cuda")


def to_host_f64(t) -> np.ndarray:
    """Device tensor -> fp64 numpy (exact upcast)."""
    import torch
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return workloads.to_f64(t.view(torch.int16).numpy().view(np.uint16), "bf16")
    return t.numpy().astype(np.float64)


def to_host_bits(t) -> np.ndarray:
    """Device tensor -> numpy array of its raw element bits."""
    import torch
    t = t.detach().to("cpu").contiguous()
    if t.element_size() == 4:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.view(torch.int16).numpy().view(np.uint16)


def host_bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.itemsize == 4 else a.view(np.uint16)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return err / scale if scale > 0 else err


def sample_indices(shape, n, rng, include_corners=True) -> np.ndarray:
    """n random (n, k, h, w) output indices, plus every corner/edge-midpoint
    of the spatial plane for a few (n, k) pairs."""
    N, K, P, Q = shape
    idx = np.stack([rng.integers(0, s, size=n) for s in shape], axis=1)
    if include_corners:
        extra = []
        for nn in {0, N - 1}:
            for kk in {0, K // 2, K - 1}:
                for hh in {0, P // 2, P - 1}:
                    for ww in {0, Q // 2, Q - 1}:
                        extra.append((nn, kk, hh, ww))
        idx = np.concatenate([idx, np.array(extra)], axis=0)
    return idx.astype(np.int64)

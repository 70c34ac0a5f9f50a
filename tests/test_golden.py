"""Fixtures printed on the pages (no GPU): each file under tests/golden/
cites the page and section it comes from."""
import os

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_fixture(name):
    vals = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, value = (s.strip() for s in line.split("=", 1))
        vals[key] = tuple(float(v) if "." in v else int(v) for v in value.split(","))
    return vals


def test_opencl_benchmarks_layer_shapes():
    g = read_fixture("opencl_benchmarks_layer.txt")
    x_shape, w_shape = g["inputs"], g["weights"]
    (s,), (p,) = g["stride"], g["padding"]
    # the printed output shape follows from the printed input, filter,
    # stride and padding through the oracle's output-extent arithmetic
    P, Q = oracle.out_dims(x_shape, w_shape, s, p, 1)
    assert (x_shape[0], w_shape[0], P, Q) == g["outputs"]
    assert g["bias"] == (w_shape[0],)
    # and it is the layer the benchmark's headline workload reproduces
    L = workloads.LAYERS["mid_3x3_fp32"]
    assert L.x_shape == x_shape and L.w_shape == w_shape
    assert L.stride == (s, s) and L.pad == (p, p) and L.b_dist is not None


def test_opencl_benchmarks_run_time_is_context_only():
    g = read_fixture("opencl_benchmarks_layer.txt")
    (ms,) = g["run_ms_normal"]
    flops = 2 * 1024 * 512 * 9 * 13 * 13
    # about 1.75 GFLOP/s on the page's mobile GPU
    assert abs(flops / (ms * 1e-3) / 1e9 - 1.746) < 0.01

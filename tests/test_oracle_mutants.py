"""The oracle's pins must catch plausible mistakes (CPU only).

Each case plants one mistake in a private copy of ``oracle/conv_oracle.c``
(a textual substitution; the committed source is untouched), compiles that
copy with gcc into a temporary directory, swaps it in for the real oracle and
runs the pin tests of ``test_oracle_pins``: at least one must fail.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "conv_oracle.c")

# (name, text in the source, replacement, occurrence to replace: None = all)
MUTANTS = [
    ("filter_flipped", "w[((k * Cg + c) * d[DR] + r) * d[DS] + q]",
     "w[((k * Cg + c) * d[DR] + (d[DR] - 1 - r)) * d[DS] + (d[DS] - 1 - q)]"),
    ("bias_dropped", "return b ? acc + b[k] : acc;", "return acc;"),
    ("pad_sign", "int64_t ih = h * d[DSH] - d[DPH] + r * d[DDH];\n                int64_t iw",
     "int64_t ih = h * d[DSH] + d[DPH] + r * d[DDH];\n                int64_t iw"),
    ("dilation_ignored_w", "int64_t iw = wo * d[DSW] - d[DPW] + q * d[DDW];",
     "int64_t iw = wo * d[DSW] - d[DPW] + q;"),
    ("stride_ignored_h", "int64_t ih = h * d[DSH] - d[DPH] + r * d[DDH];\n                int64_t iw",
     "int64_t ih = h - d[DPH] + r * d[DDH];\n                int64_t iw"),
    ("filter_transposed_kc", "w[((k * Cg + c) * d[DR] + r) * d[DS] + q]",
     "w[((c * d[DK] + k) * d[DR] + r) * d[DS] + q]"),
    ("filter_rs_swapped", "w[((k * Cg + c) * d[DR] + r) * d[DS] + q]",
     "w[((k * Cg + c) * d[DS] + q) * d[DR] + r]"),
    ("padding_not_zero", "if (ih < 0 || ih >= d[DH] || iw < 0 || iw >= d[DW]) return 0.0;",
     "if (ih < 0 || ih >= d[DH] || iw < 0 || iw >= d[DW]) return 1.0;"),
    ("extent_off_by_one", "return (padded - span) / s + 1;", "return (padded - span) / s;"),
    ("group_offset_dropped", "const int64_t c0 = (k / Kg) * Cg;", "const int64_t c0 = 0;"),
    ("repack_width_before_height", "dst = ((n * C + c) * P + h) * pitch + xc * R + r;",
     "dst = ((n * C + c) * P + h) * pitch + r * ww + xc;"),
    ("repack_hwc_channel_outer", "dst = (n * P + h) * pitch + (xc * R + r) * C + c;",
     "dst = (n * P + h) * pitch + c * ww * R + xc * R + r;"),
    ("repack_row_stride_ignored", "int64_t ih = h * d[DSH] - d[DPH] + r * d[DDH];\n                        int64_t iw = xc - d[DPW];",
     "int64_t ih = h - d[DPH] + r * d[DDH];\n                        int64_t iw = xc - d[DPW];"),
    ("repack_no_pad_shift", "int64_t iw = xc - d[DPW];", "int64_t iw = xc;"),
    ("win_width_short", "return (Q - 1) * d[DSW] + d[DDW] * (d[DS] - 1) + 1;",
     "return (Q - 1) * d[DSW] + d[DDW] * (d[DS] - 1);"),
    ("pitch_not_rounded", "return (row_elems + v - 1) / v * v;", "return row_elems;"),
    ("relu_dropped", "return relu ? fmax(v, 0.0) : v;", "return v;"),
    ("pool_min_not_max", "m = fmax(m, act(", "m = fmin(m, act("),
    ("pool_stride_one", "y[(nk * P + 2 * j + dy) * Q + 2 * i + dx]", "y[(nk * P + j + dy) * Q + i + dx]"),
    ("pool_column_dropped", "y[(nk * P + 2 * j + dy) * Q + 2 * i + dx]", "y[(nk * P + 2 * j + dy) * Q + 2 * i]"),
    ("pool_row_dropped", "y[(nk * P + 2 * j + dy) * Q + 2 * i + dx]", "y[(nk * P + 2 * j) * Q + 2 * i + dx]"),
]

PIN_TESTS = [getattr(pins, n) for n in dir(pins) if n.startswith("test_")]


def _run_pins():
    failures = []
    for t in PIN_TESTS:
        marks = getattr(t, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        cases = [()]
        if params:
            argnames = params[0].args[0]
            n = len([a.strip() for a in argnames.split(",")])
            cases = [v if n > 1 else (v,) for v in params[0].args[1]]
        for args in cases:
            try:
                t(*args)
            except Exception as e:   # noqa: BLE001 -- any failure counts as caught
                failures.append((t.__name__, type(e).__name__))
                break
    return failures


def test_real_oracle_passes_pins():
    assert _run_pins() == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    src = open(SRC).read()
    assert old in src, f"mutation site for {name} not found"
    mutated = src.replace(old, new)
    c_path = tmp_path / "mutant.c"
    c_path.write_text(mutated)
    so_path = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                           "-o", str(so_path), str(c_path), "-lm"])
    saved = oracle._lib
    oracle._lib = oracle.open_library(str(so_path))
    try:
        failures = _run_pins()
    finally:
        oracle._lib = saved
    assert failures, f"mutant {name} passed every pin"

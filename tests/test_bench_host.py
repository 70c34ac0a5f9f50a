"""Host logic of bench.py (no GPU): kernel-name shortening, trace
statistics and the roofline arithmetic."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(spec)
spec.loader.exec_module(bench)


def test_short_name():
    assert bench.short_name("_ZN3ciw12_GLOBAL__N_121conv_mfma_band_kernelIDF16_DF16_Li4EEEvPKtS3_") \
        == "conv_mfma_band_kernel"
    assert bench.short_name("_ZN3ciw19split_reduce_kernelEPKfPfi") == "split_reduce_kernel"
    assert bench.short_name("void at::native::fill(int)") == "void at::native::fill"
    assert bench.short_name("void ciw::(anonymous namespace)::conv_fp32_mfma_kernel<true, 2>"
                            "(float const*, float*)") == "conv_fp32_mfma_kernel"
    assert bench.is_library_kernel("void ciw::(anonymous namespace)::k<1>(int)")
    assert not bench.is_library_kernel("void at::native::fill(int)")


def test_trace_stats():
    calls = [[("a", 0.0, 10.0), ("b", 12.0, 3.0)],
             [("a", 100.0, 8.0), ("b", 109.0, 5.0)],
             [("a", 200.0, 9.0), ("b", 210.0, 4.0)]]
    st = bench.trace_stats(calls)
    assert st["calls"] == 3
    assert st["kernels"]["a"] == {"best_us": 8.0, "median_us": 9.0}
    assert st["kernels"]["b"] == {"best_us": 3.0, "median_us": 4.0}
    assert st["kernel_sum"] == {"best_us": 13.0, "median_us": 13.0}
    # span: first start to last end
    assert st["span"] == {"best_us": 14.0, "median_us": 14.0}
    assert st["dominant"] == "a"
    # a kernel launched twice in one call is keyed by position
    st2 = bench.trace_stats([[("a", 0.0, 1.0), ("a", 2.0, 2.0)]])
    assert set(st2["kernels"]) == {"a#0", "a#1"}


def test_roofline_entry():
    # an fp16 MFMA kernel above the ridge: compute bound, against 2516.6
    r = bench.roofline_entry(flops=int(2516.6e12 * 1e-3), nbytes=1000, dtype="f16",
                             dominant="conv_mfma_band_kernel", ms=2.0)
    assert r["bound"] == "mfma" and r["peak"] == 2516.6
    assert r["frac"] == pytest.approx(0.5, abs=1e-4)
    # below the ridge: HBM bound, with the compute fraction still given
    r = bench.roofline_entry(flops=10 ** 9, nbytes=8 * 10 ** 9, dtype="f16",
                             dominant="conv_mfma_rows_kernel", ms=2.0)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["frac"] == pytest.approx(0.5, abs=1e-4)
    assert r["compute_unit"] == "mfma"
    # fp32 VALU kernel: the vector peak, labelled alu
    r = bench.roofline_entry(flops=int(157.3e12 * 1e-3), nbytes=1000, dtype="f32",
                             dominant="conv_fp32_klanes_kernel", ms=1.0)
    assert r["bound"] == "alu" and r["frac"] == pytest.approx(1.0, abs=1e-4)
    # fp32 matrix-core kernel: the fp32 MFMA peak (157.3), labelled mfma
    r = bench.roofline_entry(flops=int(157.3e12 * 1e-3), nbytes=1000, dtype="f32",
                             dominant="conv_fp32_mfma_kernel", ms=1.0)
    assert r["bound"] == "mfma" and r["peak"] == 157.3
    # depthwise is bound by HBM whatever its intensity
    r = bench.roofline_entry(flops=10 ** 12, nbytes=10 ** 6, dtype="f32",
                             dominant="conv_dw_block_kernel", ms=1.0)
    assert r["bound"] == "hbm"

"""CPU sanitizer builds (AddressSanitizer + UndefinedBehaviorSanitizer).

  * the oracle (oracle/conv_oracle.c) built with gcc and every entry point
    driven over edge-case layers (tests/sanitize/oracle_driver.c), plus a
    copy of the oracle with one planted out-of-bounds write, which the
    sanitized build must stop;
  * the library's host code -- descriptor validation, output extents,
    window geometry, workspace and chunk arithmetic, kernel plans -- built
    with hipcc, sanitizers on the host pass only, and driven through the C
    ABI over thousands of valid, edge and wrapping descriptors
    (tests/sanitize/abi_driver.cpp).  Its heavy per-type kernel files are
    linked from the library's own build.

CPU only: skipped where a GPU is visible (the drivers never launch a
kernel there either)."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "cnn_convolution_im2win_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
HIPCC = "/opt/rocm/bin/hipcc"

if os.path.exists("/dev/kfd"):
    pytest.skip("a GPU is visible: the sanitizer builds run on the CPU only", allow_module_level=True)

ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
GCC_SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all"]
# sanitizers on the host pass only: each flag right after -Xarch_host
HIP_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _gcc_oracle(tmp, src):
    exe = os.path.join(tmp, "oracle_driver")
    subprocess.run(["gcc", "-std=c99"] + GCC_SAN + ["-o", exe, os.path.join(HERE, "oracle_driver.c"),
                    src, "-lm"], check=True, capture_output=True, text=True)
    return exe


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = _gcc_oracle(str(tmp_path), os.path.join(ROOT, "oracle", "conv_oracle.c"))
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "clean" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_sanitized_oracle_build_catches_a_planted_overrun(tmp_path):
    """The same build on a copy of the oracle whose unpooled epilogue runs
    one element past the output must fail with a sanitizer report."""
    src = open(os.path.join(ROOT, "oracle", "conv_oracle.c")).read()
    planted = "for (int64_t i = 0; i <= N * K * P * Q; ++i) out[i] = act(y[i], relu);"
    mutant = src.replace("for (int64_t i = 0; i < N * K * P * Q; ++i) out[i] = act(y[i], relu);", planted)
    assert mutant != src
    path = os.path.join(str(tmp_path), "conv_oracle_planted.c")
    with open(path, "w") as f:
        f.write(mutant)
    exe = _gcc_oracle(str(tmp_path), path)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr


# the library sources whose host code is rebuilt with the sanitizers (the
# rest are per-type kernel instantiations, linked from the library's build)
SAN_SOURCES = ["api.cpp", "transform.hip", "conv_fp32.hip", "conv_fp32_mfma.hip", "conv_mfma.hip",
               "conv_dw.hip", "conv_dw_implicit.hip", "conv_implicit.hip"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="no hipcc")
def test_host_abi_under_sanitizers(tmp_path):
    from cnn_convolution_im2win_amd import build
    others = [s for s in build.SOURCES if s not in SAN_SOURCES]
    objs_main = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in others]
    if not all(os.path.exists(o) for o in objs_main):
        pytest.skip("the library is not built (run cnn_convolution_im2win_amd.build)")
    tmp = str(tmp_path)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    base = [HIPCC, f"--offload-arch={build.ARCH}", "-std=c++17", "-fPIC", "-g", "-O1",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + HIP_SAN + inc

    def compile_one(src):
        out = os.path.join(tmp, os.path.splitext(os.path.basename(src))[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        r = subprocess.run(base + lang + ["-c", src, "-o", out], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return out

    srcs = [os.path.join(CSRC, s) for s in SAN_SOURCES] + [os.path.join(HERE, "abi_driver.cpp")]
    with ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = os.path.join(tmp, "abi_driver")
    r = subprocess.run([HIPCC, f"--offload-arch={build.ARCH}"] + HIP_SAN[:4] + ["-o", exe] + objs + objs_main,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-3000:])
    assert "clean" in r.stdout

"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
the C oracle driven on small inputs (tests/sanitize/oracle_driver.c), and the
C ABI layer (csrc/gq_api.cpp: checks, table planning, workspace layout) with
counting stand-ins for its device launchers (tests/sanitize/api_stubs.cpp)
driven through every entry point and refusal (tests/sanitize/api_driver.cpp).
Both are built with g++/gcc for the host only; no GPU code is involved."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g",
       "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr)
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_driver")
        _run(["gcc", "-std=c11", "-ffp-contract=off", *SAN, "-o", exe,
              os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
              os.path.join(ROOT, "oracle", "oracle.c"), "-lm"], d)
        assert "all checks passed" in _run([exe], d)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers not available")
def test_c_abi_layer_under_asan_ubsan():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "api_driver")
        inc = ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
               "-I" + os.path.join(ROOT, "quantized_unpack_q4_amd", "csrc")]
        srcs = [os.path.join(ROOT, "tests", "sanitize", "api_driver.cpp"),
                os.path.join(ROOT, "tests", "sanitize", "api_stubs.cpp"),
                os.path.join(ROOT, "quantized_unpack_q4_amd", "csrc", "gq_api.cpp")]
        _run(["g++", "-std=c++17", *SAN, *inc, "-o", exe, *srcs, "-L/opt/rocm/lib", "-lamdhip64",
              "-Wl,-rpath,/opt/rocm/lib"], d)
        assert "all checks passed" in _run([exe], d)

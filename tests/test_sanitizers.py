"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Two CPU-only builds, made in a temporary directory and run once:
  * the oracle (oracle/oracle.c) with tests/sanitize/oracle_driver.c, gcc
    -fsanitize=address,undefined;
  * the library's host code -- argument checks of every entry point
    (twd_api.hip), the width dispatch, the weight format (format_host.cpp)
    and the sweep planner (sweep_plan.cpp) -- with tests/sanitize/
    host_driver.cpp, built host-only by hipcc with the sanitizers on the host
    side and the device launches replaced by tests/sanitize/host_stubs.cpp.
Any sanitizer report aborts the driver (no recovery), which fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ternary_weight_decode_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, env=ENV)
    assert r.returncode == 0, f"{' '.join(cmd[:3])}...\n{r.stdout}\n{r.stderr[-4000:]}"
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc missing")
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-g", "-O1", "-fopenmp",
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(SAN, "oracle_driver.c"),
          "-lm", "-o", exe], str(tmp_path))
    assert "oracle driver: ok" in _run([exe], str(tmp_path))


def test_library_host_code_under_sanitizers(tmp_path):
    if not shutil.which("hipcc"):
        pytest.skip("hipcc missing")
    exe = str(tmp_path / "host_driver")
    srcs = [os.path.join(CSRC, f) for f in ("twd_api.hip", "dispatch.hip", "format_host.cpp",
                                            "sweep_plan.cpp")]
    srcs += [os.path.join(SAN, "host_stubs.cpp"), os.path.join(SAN, "host_driver.cpp")]
    _run(["hipcc", "-x", "hip", "--cuda-host-only", "-std=c++17",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all", "-g", "-O1", *srcs, "-o", exe],
         str(tmp_path))
    assert "host driver: ok" in _run([exe], str(tmp_path))

"""The C ABI's host code (fp8_scaled_gemm_amax_amd/csrc/api.cpp: argument
validation, the device-properties cache, dispatch) built with g++ under the
address and undefined-behaviour sanitizers and driven by
tests/api_sanitize_driver.cpp, which replaces the kernel launchers and HIP's
device queries with stubs (one gfx950 device) and calls every entry point with
valid and invalid arguments. CPU only; skipped without g++, the HIP headers or
the sanitizer runtimes."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIP_INCLUDE = "/opt/rocm/include"


def test_api_host_code_under_sanitizers(tmp_path):
    if shutil.which("g++") is None or not os.path.isdir(HIP_INCLUDE):
        pytest.skip("no g++ or no HIP headers")
    exe = str(tmp_path / "api_sanitized")
    flags = ["-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I" + HIP_INCLUDE,
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    srcs = [os.path.join(ROOT, "tests", "api_sanitize_driver.cpp"),
            os.path.join(ROOT, "fp8_scaled_gemm_amax_amd", "csrc", "api.cpp")]
    build = subprocess.run(["g++", *flags, "-o", exe, *srcs, "-lpthread"], capture_output=True, text=True)
    if build.returncode != 0 and ("asan" in build.stderr.lower() or "ubsan" in build.stderr.lower()):
        pytest.skip("sanitizer runtime not available: " + build.stderr[-200:])
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
    assert "every check passed" in run.stdout

"""The CPU oracle's C code under the address and undefined-behaviour
sanitizers: tests/oracle_sanitize_driver.c calls every entry point on ragged
shapes and special values (NaN, Inf, zeros, bf16 subnormals, saturating
values), and any invalid access or undefined operation aborts the run. CPU only;
needs gcc with libasan / libubsan (skipped otherwise)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    exe = str(tmp_path / "oracle_sanitized")
    flags = ["-O1", "-g", "-std=c11", "-fno-omit-frame-pointer", "-fno-fast-math", "-ffp-contract=off",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    build = subprocess.run(["gcc", *flags, "-o", exe, os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"),
                            os.path.join(ROOT, "oracle", "fp8_oracle.c"), "-lm"], capture_output=True, text=True)
    if build.returncode != 0 and ("asan" in build.stderr.lower() or "ubsan" in build.stderr.lower()):
        pytest.skip("sanitizer runtime not available: " + build.stderr[-200:])
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]

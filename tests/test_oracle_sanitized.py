"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only), driven through every entry point on small and
edge-case shapes by oracle/sanitize_driver.c: an access outside an array or
an undefined operation in the oracle aborts the driver."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-O1", "-g", "-std=gnu11", "-fopenmp", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer",
           os.path.join(ROOT, "oracle", "qlin_oracle.c"),
           os.path.join(ROOT, "oracle", "sanitize_driver.c"), "-o", exe, "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "sanitizer" in build.stderr.lower():
        pytest.skip(f"sanitizer runtime unavailable: {build.stderr[-300:]}")
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failures" in run.stdout

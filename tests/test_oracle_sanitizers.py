"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc, host
code only) and driven through every entry point, valid and invalid arguments alike
(tests/sanitize/oracle_driver.c).  The pages warn that invalid group sizes corrupt or crash
memory accesses ("Group-GEMM in XLA", Part 2); the oracle's clamping reading must stay in
bounds."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-O1", "-g", "-fopenmp", "-std=c11", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
           "-o", exe, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in r.stderr.lower():
        pytest.skip("the sanitizer runtime is not installed: " + r.stderr[-200:])
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="4")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failures" in run.stdout

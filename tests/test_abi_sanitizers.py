"""The C ABI's host-side argument checks (api.hip) built with AddressSanitizer and
UndefinedBehaviorSanitizer on the host and driven with refused and random arguments
(tests/sanitize/abi_driver.cpp).  CPU only: the driver passes fake addresses, so it refuses to
run where a GPU is visible, and every call that passes validation fails at its first runtime
call instead of launching."""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "group_gemm_amd", "csrc")
OBJ = os.path.join(ROOT, "group_gemm_amd", "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_abi_validation_under_asan_and_ubsan(tmp_path):
    kernels = [o for o in glob.glob(os.path.join(OBJ, "*.hip.o")) if not o.endswith("api.hip.o")]
    if not kernels:
        pytest.skip("the library has not been built (python -m group_gemm_amd.build)")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-w", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    api_o = str(tmp_path / "api_san.o")
    r = subprocess.run([HIPCC, *common, *san, "-c", os.path.join(CSRC, "api.hip"), "-o", api_o], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    drv_o = str(tmp_path / "abi_driver.o")
    r = subprocess.run([HIPCC, *common, *san, "-c", os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", drv_o],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "abi_driver")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *san, drv_o, api_o, *kernels, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=900)
    if run.returncode == 77:
        pytest.skip(run.stdout.strip())
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-3000:]
    assert "0 failures" in run.stdout

"""The C ABI's host-side argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

bsta_api.hip is compiled for the host alone (no device code) with the
sanitizers, linked with launcher stubs and a driver that calls every entry
point with valid and invalid arguments (tests/host_sanitize/).  The driver
checks return codes, that rejected calls never reach a launcher, and the
thread-local error detail; the sanitizers abort on any memory error or
undefined behaviour in the validation code.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_validation_under_asan_ubsan(tmp_path):
    src = os.path.join(ROOT, "tests", "host_sanitize")
    exe = str(tmp_path / "abi_host_check")
    cmd = [HIPCC, "-x", "hip", "--offload-host-only", *SAN, "-fno-omit-frame-pointer", "-g", "-O1",
           "-std=c++17", f"-I{ROOT}/include", f"-I{ROOT}/block_sparse_tiled_amd/csrc",
           os.path.join(ROOT, "block_sparse_tiled_amd", "csrc", "bsta_api.hip"),
           os.path.join(src, "stubs.cpp"), "-x", "c++", os.path.join(src, "driver.cpp"),
           "-o", exe, "-lpthread"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("LD_PRELOAD", None) if "LD_PRELOAD" in env and "asan" in env["LD_PRELOAD"] else None
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert run.stdout.startswith("OK "), run.stdout
    assert "ERROR: AddressSanitizer" not in run.stderr and "runtime error" not in run.stderr

"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
the C oracle over every format and function on exactly sized buffers, and the
C ABI's argument checking with the kernel launchers replaced by stubs (valid,
invalid and int64-overflowing shapes, workspaces).  The drivers live in
tests/native/; each run has a time limit."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd_build, exe, tmp_path):
    r = subprocess.run(cmd_build, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env, cwd=tmp_path)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_driver"
    out = _run(["gcc", "-std=gnu11", *SAN, os.path.join(HERE, "native", "oracle_driver.c"),
                os.path.join(ROOT, "oracle", "oracle.c"), "-o", str(exe), "-lm"], exe, tmp_path)
    assert "oracle driver: ok" in out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers not available")
def test_api_argument_checks_under_sanitizers(tmp_path):
    exe = tmp_path / "api_host_driver"
    out = _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "quantized_dequant_matrix_amd", "csrc"),
                os.path.join(HERE, "native", "api_host_driver.cpp"),
                os.path.join(ROOT, "quantized_dequant_matrix_amd", "csrc", "qmv_api.cpp"), "-o", str(exe)], exe, tmp_path)
    assert "api host driver: ok" in out

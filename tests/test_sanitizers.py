"""Host sanitizer builds (no GPU): the C oracle under AddressSanitizer +
UndefinedBehaviorSanitizer and under ThreadSanitizer (its row pool shares a
work counter), and the C-ABI front end's argument validation (api.cpp and
plan.cpp with the kernel launchers stubbed) under the same three."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "autoregressive_video_diffusion_amd", "csrc")

ASAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
TSAN = ["-fsanitize=thread"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
           TSAN_OPTIONS="halt_on_error=1")


def _run(cmd, tmp_path, name):
    exe = str(tmp_path / name)
    r = subprocess.run(cmd + ["-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "ok" in r.stdout
    assert "Sanitizer" not in r.stderr, r.stderr[-4000:]


@pytest.mark.parametrize("san", ["asan_ubsan", "tsan"])
def test_oracle_under_sanitizer(tmp_path, san):
    flags = ASAN if san == "asan_ubsan" else TSAN
    cmd = ["gcc", "-std=c11", "-O1", "-g", *flags, os.path.join(ROOT, "oracle", "oracle.c"),
           os.path.join(HERE, "oracle_driver.c"), "-lm", "-lpthread"]
    _run(cmd, tmp_path, f"oracle_{san}")


@pytest.mark.skipif(not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"),
                    reason="HIP headers not installed")
@pytest.mark.parametrize("san", ["asan_ubsan", "tsan"])
def test_abi_validation_under_sanitizer(tmp_path, san):
    flags = ASAN if san == "asan_ubsan" else TSAN
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           *flags, os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(HERE, "launch_stubs.cpp"), os.path.join(HERE, "abi_driver.cpp"),
           "-lpthread"]
    _run(cmd, tmp_path, f"abi_{san}")

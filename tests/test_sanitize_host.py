"""The C ABI's host-side validation (api*.cpp, profile.cpp) built with g++
under AddressSanitizer and UndefinedBehaviorSanitizer, linked against
launcher stand-ins (tests/sanitize/stubs.cpp), and driven through every
entry point with valid and invalid arguments (tests/sanitize/driver.cpp).
CPU only: no kernel runs."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "diffusion_augmented_decoding_amd", "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("api.cpp", "api_layer.cpp", "api_step.cpp", "profile.cpp")] + \
          [os.path.join(HERE, "sanitize", f) for f in ("stubs.cpp", "driver.cpp")]


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include")] + SOURCES + ["-L/opt/rocm/lib", "-lamdhip64",
                                                          "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "launches reached" in r.stdout

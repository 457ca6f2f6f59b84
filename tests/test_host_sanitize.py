"""CPU: the host side of the C ABI (plan.cpp, api.cpp) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer, with stub kernel launchers that
check every launch's parameters against its plan (tests/host_sanitize/driver.cpp).
No GPU code is built or run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = "/opt/rocm"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the ROCm headers")
def test_host_library_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "host_sanitize"
    csrc = os.path.join(ROOT, "speculative_verify_kv_amd", "csrc")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include", f"-I{csrc}",
           os.path.join(csrc, "plan.cpp"), os.path.join(csrc, "api.cpp"),
           os.path.join(ROOT, "tests", "host_sanitize", "driver.cpp"),
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stdout + build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout[-4000:] + run.stderr[-4000:]
    assert run.stdout.startswith("ok "), run.stdout
    assert int(run.stdout.split()[1]) > 1000

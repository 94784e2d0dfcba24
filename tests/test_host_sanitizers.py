"""The host side of the C ABI (argument checks, planners, RoPE table) built
with AddressSanitizer and UndefinedBehaviorSanitizer by g++, kernels replaced
by counting stand-ins (tests/host/), and run on the CPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_latent_kv_04_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")
ROCM_INC = "/opt/rocm/include"


@pytest.mark.timeout(300)
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(ROCM_INC):
        pytest.skip("g++ or the ROCm headers are missing")
    exe = str(tmp_path / "sanitize_driver")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM_INC}", f"-I{os.path.join(ROOT, 'include')}",
           f"-I{CSRC}",
           os.path.join(CSRC, "mla_api.cpp"), os.path.join(CSRC, "produce_api.cpp"),
           os.path.join(HOST, "launch_stubs.cpp"), os.path.join(HOST, "sanitize_driver.cpp"),
           "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    # verify_asan_link_order=0: the environment may preload a library ahead of
    # the sanitizer runtime
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=240)
    assert run.returncode == 0, (run.stdout[-3000:], run.stderr[-3000:])
    assert run.stdout.strip().endswith("ok")

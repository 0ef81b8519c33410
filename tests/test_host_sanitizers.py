"""The host layer (host.cpp: layouts, codebook, validation, dispatch) built host-only with
the address and undefined-behaviour sanitizers and driven through every entry point on the
CPU, against link-time stand-ins for the kernel launchers and the HIP device queries
(tests/host_asan/). No GPU code is built or run."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ not found")
def test_host_layer_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "host_asan")
    here = os.path.join(ROOT, "tests", "host_asan")
    cmd = [CLANG, "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "agent_q8_quant_amd", "csrc"),
           "-I" + here, "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g", "-O1",
           os.path.join(ROOT, "agent_q8_quant_amd", "csrc", "host.cpp"),
           os.path.join(here, "stubs.cpp"), os.path.join(here, "driver.cpp"), "-o", exe]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "all checks passed" in r.stdout

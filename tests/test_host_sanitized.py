"""The host side of the C ABI (validation, layout, launch planning) under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

tests/host/abi_host_driver.cpp drives every host path that needs no device
(sizes at and past their limits, every rejected call, the launch tiles) and
is linked with moe_ep_api.cpp and moe_ep_plan.cpp, built by g++ with both
sanitizers; the kernel launchers are stubs that the driver must not reach.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "combine_token_dest_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_host_paths_clean_under_sanitizers():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "abi_host_driver")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
               "-I", CSRC, os.path.join(ROOT, "tests", "host", "abi_host_driver.cpp"),
               os.path.join(CSRC, "moe_ep_api.cpp"), os.path.join(CSRC, "moe_ep_plan.cpp"),
               "-L", os.path.join(ROCM, "lib"), "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lamdhip64", "-o", exe]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        p = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert p.returncode == 0, p.stdout + p.stderr
        assert "fails 0" in p.stdout
        assert "reached" not in p.stdout
        assert "runtime error" not in p.stderr and "AddressSanitizer" not in p.stderr

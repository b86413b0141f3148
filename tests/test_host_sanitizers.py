"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): csrc/api.cpp and csrc/plan.cpp are built with g++ beside the
driver tests/asan/abi_fuzz.cpp, which stubs the HIP runtime queries and the
kernel launchers and sweeps seeded valid and invalid call shapes through the
planner, the workspace-size queries and the decode entry points, checking
each plan a launch would receive against what the kernels assume.  Any
sanitizer report, failed invariant or unexpected status fails the test."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the ROCm headers")
def test_abi_sweep_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I" + ROCM_INCLUDE,
           os.path.join(ROOT, "tests", "asan", "abi_fuzz.cpp"),
           os.path.join(ROOT, "paged_kv_decode_block_amd", "csrc", "api.cpp"),
           os.path.join(ROOT, "paged_kv_decode_block_amd", "csrc", "plan.cpp"),
           "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe, "200000"], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "abi sweep ok" in run.stdout
    launches = int(run.stdout.split("shapes, ")[1].split(" launches")[0])
    assert launches > 10000, run.stdout

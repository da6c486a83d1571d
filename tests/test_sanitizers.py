"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/native/abi_sanitize.cpp drives the validation of every entry point,
the workspace sizing over a range of shapes and the host Stochastic Length
sampler on random batches. It is built here with g++ (host code only: the
device launchers are stubs that abort if reached) together with api.cpp,
plan.cpp and sampler.cpp, and must exit cleanly with no sanitizer report."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hstu_sequential_transducer_jagged_amd", "csrc")
NATIVE = os.path.join(ROOT, "tests", "native")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or
                    not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")),
                    reason="needs g++ and the HIP runtime library")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "abi_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(NATIVE, "abi_sanitize.cpp"), os.path.join(NATIVE, "launch_stubs.cpp"),
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(CSRC, "sampler.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-lamdhip64", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    print(r.stdout)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stderr
    assert "runtime error" not in r.stderr
    assert "all host checks passed" in r.stdout

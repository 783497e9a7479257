"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tq_api.cpp and tq_codebook.cpp are compiled for the host with the ROCm clang
and -fsanitize=address,undefined, linked with host stand-ins for the HIP
runtime and for the kernel launchers (tests/host_sanitize/fake_runtime.cpp),
and driven through every entry point, error paths and successful paths, by
tests/host_sanitize/driver.cpp.  No GPU is involved: the point is the host
logic (argument checks, size queries, the R / S images of tq_create, the
codebook tables, workspace partitions), where any out-of-bounds access,
use after free, leak or undefined operation fails the run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"
SOURCES = [os.path.join(ROOT, "kv_cache_vector_compress_amd", "csrc", "tq_api.cpp"),
           os.path.join(ROOT, "kv_cache_vector_compress_amd", "csrc", "tq_codebook.cpp"),
           os.path.join(ROOT, "tests", "host_sanitize", "fake_runtime.cpp"),
           os.path.join(ROOT, "tests", "host_sanitize", "driver.cpp")]


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not installed")
def test_abi_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "tq_host_sanitize")
    cmd = [CLANG, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", *SOURCES, "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-6000:]
    assert "Sanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert out.rstrip().endswith("ok"), out[-2000:]
    print(out.splitlines()[-2])

"""The host block manager (csrc/pa_blocks.cpp: the free-block ring, reference
counts, block lists and the step-metadata builder) built on its own with
AddressSanitizer and UndefinedBehaviorSanitizer (g++, host code only), and
tests/test_block_manager.py run against that build in a child process, so an
out-of-bounds index, a use after free or undefined arithmetic in it stops the
run.  The address-space-limit test is left out there: the sanitizer's shadow
memory reserves far more address space than that limit allows."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "paged_kv_cache_token_amd", "csrc", "pa_blocks.cpp")


def _runtime(gxx: str, name: str):
    p = subprocess.run([gxx, f"-print-file-name={name}"], capture_output=True,
                       text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_block_manager_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    asan, ubsan = _runtime(gxx, "libasan.so"), _runtime(gxx, "libubsan.so")
    if not asan or not ubsan:
        pytest.skip("g++ has no sanitizer runtimes")
    lib = str(tmp_path / "libpa_blocks_sanitized.so")
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-shared", "-fPIC", "-I", os.path.join(ROOT, "include"), SRC, "-o", lib],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", PA_TEST_BLOCKS_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        "-k", "not host_allocation_failure",
                        os.path.join(ROOT, "tests", "test_block_manager.py")],
                       env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, out
    assert " passed" in r.stdout, out

"""The host block manager's C++ under AddressSanitizer and UndefinedBehaviorSanitizer.

``pa_block_manager.cpp`` is host-only code (free list, intrusive LRU lists,
hash maps, swap state).  This test compiles it with g++ and
``-fsanitize=address,undefined`` into a separate shared library (no GPU code
is involved), then runs the whole block-manager suite
(tests/test_block_manager.py: the pinned model, the library compared with it
operation by operation on random traces of 16- and 8-token blocks, the error
paths) in a child process whose manager calls go to that build
(``PA_BM_LIBRARY``), with the ASan runtime preloaded and every report fatal.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "paged_kv_cache_365_amd", "csrc", "pa_block_manager.cpp")


def test_block_manager_suite_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ is not installed")
    lib = str(tmp_path / "libpa_bm_sanitized.so")
    build = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fPIC", "-shared",
             "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
             "-D__HIP_PLATFORM_AMD__", SRC, "-o", lib]
    r = subprocess.run(build, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    assert os.path.exists(asan), "the ASan runtime is missing"
    env = dict(os.environ)
    env.update({
        "PA_BM_LIBRARY": lib,
        "LD_PRELOAD": asan,
        # CPython keeps objects alive at exit by design: leak reports would be noise
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_block_manager.py"),
           "-q", "-x", "-p", "no:cacheprovider"]
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=str(tmp_path),
                       timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out and "failed" not in out, out[-2000:]

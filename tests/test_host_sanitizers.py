"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
kvq_api.cpp (argument validation, pool layout, page bookkeeping) is rebuilt by
g++ with both sanitizers, linked with this build's device objects, and the CPU
tests of the ABI (every error path, struct layouts, plan sizes) run against it
in a child process with the ASan runtime preloaded. Any heap or stack error,
use after free, signed overflow, misaligned access or other undefined
behaviour aborts the child and fails this test."""

import os
import subprocess
import sys

import pytest

from bit_kv_cache_groupwise_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_cpu_tests_pass_under_asan_and_ubsan(tmp_path):
    if not all(os.path.exists(os.path.join(B.BUILD, u[1])) for u in B.units() if u[3]):
        pytest.skip("device objects not built here")
    lib = B.build_host_sanitized(str(tmp_path))
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    preload = " ".join(p for p in (asan, os.environ.get("LD_PRELOAD", "")) if p)  # the ASan runtime first
    env = dict(os.environ, LD_PRELOAD=preload, KVQ_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out

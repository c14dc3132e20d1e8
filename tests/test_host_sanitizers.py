"""The C ABI's host code (validation, workspace planning, chunk map, error
paths) under AddressSanitizer and UndefinedBehaviorSanitizer.

kda_api.cpp is built for the host only, with stand-in launchers, and the CPU
ABI tests run against that build in a child process with the sanitizer
runtime preloaded; any report aborts the child and fails this test."""
import os
import subprocess
import sys

import pytest

from chunkwise_kimi_delta_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_run_clean_under_asan_and_ubsan():
    try:
        lib = build.build_host_sanitized()
        rt = build.asan_runtime()
    except RuntimeError as e:          # no ROCm toolchain on this machine
        pytest.skip(str(e))
    env = dict(os.environ, KDA_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "Sanitizer" not in out, out[-4000:]

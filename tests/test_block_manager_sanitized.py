"""The C++ block manager under AddressSanitizer and UndefinedBehaviorSanitizer
(host code only: block_manager.cpp and status.cpp built with g++ by
paged_kv_cache_421_amd/build.py).  The random-script tests of
tests/test_library_host.py -- C++ manager against the oracle's after every
operation, with appends, forks, frees, batch appends, swapping and prefix
caching -- run in a child process whose block manager is the sanitized
build, with three times their usual length: 127 500 operations in all.  Any
invalid memory access or undefined behaviour aborts the child."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "paged_kv_cache_421_amd"))
import build as _build  # noqa: E402


def _runtime(name):
    out = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_random_scripts_under_address_and_ub_sanitizers():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("g++ has no AddressSanitizer runtime")
    if not os.path.exists(_build.HOST_SAN_LIB):
        _build.build_host_sanitized()
    env = dict(os.environ,
               LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:malloc_context_size=2:quarantine_size_mb=64",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               PAGEDKV_HOST_LIB=_build.HOST_SAN_LIB,
               PAGEDKV_SCRIPT_SCALE="3")
    # the child's block manager must be the sanitized build
    probe = subprocess.run([sys.executable, "-c",
                            "import paged_kv_cache_421_amd._lib as L; print(L.host_lib._name)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0 and probe.stdout.strip() == _build.HOST_SAN_LIB, \
        probe.stdout + probe.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-n", "4", os.path.join(ROOT, "tests", "test_library_host.py"),
                        "-k", "matches_oracle", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "14 passed" in r.stdout, tail
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, tail

"""The host runtime under AddressSanitizer and UndefinedBehaviorSanitizer.

libpkv_san.so links the same kernel objects as libpkv.so with a copy of the
host runtime (page allocator with reference counts, request caches, forks
and copy on write, the token transaction, split plans) compiled with both
sanitizers; device code is not instrumented.  The whole host-only suite
(tests/test_abi_host.py: every ABI argument check and the random
begin/append/commit/abort/reset/grow/fork/destroy schedules against the
oracle's transaction model) runs in a child process that preloads the
sanitizer runtime and loads that build, and must finish with no report.
CPU only: host-only pools never touch a device.
"""
from __future__ import annotations

import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    path = os.path.join(ROOT, "paged_kv_cache_attention_amd", "build.py")
    spec = importlib.util.spec_from_file_location("pkv_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _sanitized_env(build):
    lib = build.LIBPKV_SAN
    if not os.path.exists(lib):
        build.build_libpkv()            # also links the sanitized copy
    runtime = build.asan_runtime()
    if not os.path.exists(runtime):
        pytest.skip(f"no sanitizer runtime at {runtime}")
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": runtime,
        # Python itself is not built with the sanitizer: its allocations at
        # exit are not the library's leaks.
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "PKV_LIBRARY": lib,
    })
    return env, lib


def test_host_suite_runs_clean_under_address_and_undefined_sanitizers():
    build = _build_module()
    env, lib = _sanitized_env(build)
    probe = subprocess.run(
        [sys.executable, "-c",
         "import paged_kv_cache_attention_amd as p; "
         "maps = open('/proc/self/maps').read(); "
         "print(p.LIB_PATH, 'libpkv_san.so' in maps, 'asan' in maps)"],
        env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert probe.stdout.split() == [lib, "True", "True"], probe.stdout
    run = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
         os.path.join("tests", "test_abi_host.py")],
        env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    report = run.stdout[-4000:] + run.stderr[-4000:]
    assert run.returncode == 0, report
    assert "passed" in run.stdout and "failed" not in run.stdout, report
    for marker in ("AddressSanitizer", "runtime error:", "UndefinedBehaviorSanitizer"):
        assert marker not in run.stderr and marker not in run.stdout, report

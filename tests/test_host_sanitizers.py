"""The host library code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only): tests/test_abi.py, which drives the argument checks, the ring and sink state
rules and the step/chain validation through the C ABI, runs in a child process
against a build of la_api.cpp instrumented for the host, with the sanitizer runtime
preloaded; any report aborts the child and fails this test."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_asan_and_ubsan(tmp_path):
    from streaming_causal_video_amd import build as B
    lib = B.build_host_sanitized(str(tmp_path))
    env = dict(os.environ)
    env.update(LA_TEST_LIB_PATH=lib, LD_PRELOAD=B.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                          "-q", "-s", "-p", "no:cacheprovider"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    report = res.stdout[-3000:] + res.stderr[-3000:]
    assert res.returncode == 0, report
    assert "runtime error" not in res.stdout + res.stderr, report
    assert "AddressSanitizer" not in res.stdout + res.stderr, report
    assert " passed" in res.stdout, report

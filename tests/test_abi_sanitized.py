"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

rss_api.cpp is built for the host only with both sanitizers (errors abort) and
driven by tests/c_abi/abi_host_check.cpp: every validation error of every
entry point, binding with null and misaligned buffers, buffer sizes, the
verify / rollback call order, empty batches, and the arguments the dispatch
hands to the kernel launchers (stubbed: nothing is launched). The run must
pass every check with no sanitizer report."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "c_abi"))

import build_host_check  # noqa: E402


def test_abi_host_code_is_clean_under_asan_and_ubsan():
    exe = build_host_check.build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "Sanitizer" not in out and "runtime error" not in out, out
    assert "abi host checks passed" in r.stdout

"""The C ABI tests again, against the host-sanitized build of the library.

lib/libkda_hostsan.so links the same kernel objects with the C ABI layer
(argument validation and dispatch) compiled with AddressSanitizer and
UndefinedBehaviorSanitizer for the host.  tests/test_abi.py runs in a child
process that loads it (KDA_LIBRARY) with the sanitizer runtime preloaded; any
sanitizer report aborts that process and fails this test.  No GPU is needed:
every call is rejected, or returns, before it reaches HIP.
"""

import os
import subprocess
import sys

import pytest

from gated_delta_rule_76_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_host_sanitizers():
    runtime = build.sanitizer_runtime()
    if runtime is None:
        pytest.skip("no AddressSanitizer runtime in this ROCm install")
    if not os.path.exists(build.SAN_LIB):
        pytest.skip("the host-sanitized library is not built (python -m gated_delta_rule_76_amd.build)")
    env = dict(os.environ, KDA_LIBRARY=build.SAN_LIB, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "passed" in r.stdout

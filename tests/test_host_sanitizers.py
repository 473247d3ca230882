"""The C ABI's host-side argument checks (tests/test_api_host.py) run again against a build of
the library whose host code (psa_api.cpp) carries AddressSanitizer and UndefinedBehaviorSanitizer
(built by the package's build step into _build/libpsa_hostsan.so). Every bad argument, empty
problem and workspace query of those tests then runs under both sanitizers: an out-of-bounds
read, a use of freed memory, a signed overflow or a misaligned access in the checks aborts the
run. No GPU is used; device code is never built with a sanitizer.
"""
import os
import subprocess
import sys

from video_transformers_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))


def test_api_checks_under_host_sanitizers():
    lib = B.HOSTSAN_LIB
    if not os.path.exists(lib):
        B.build_host_sanitized()
    env = dict(os.environ)
    env.update(PSA_LIBRARY=lib, LD_PRELOAD=B.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(HERE, "test_api_host.py")],
                       env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail, tail
    assert "runtime error" not in tail, tail

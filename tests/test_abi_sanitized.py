"""The C ABI's host-side code under AddressSanitizer and
UndefinedBehaviorSanitizer.  The library is rebuilt with host-only
instrumentation (device code unchanged) and the ABI checks of
tests/test_abi.py run against it in a child process with clang's ASan
runtime preloaded; any sanitizer report aborts the child and fails the test.
No GPU is used: every call there fails validation before a launch."""

import os
import subprocess
import sys

import pytest

from sparse_long_context_query_amd import build_lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    rt = build_lib.sanitizer_runtime()
    if not rt:
        pytest.skip("clang's ASan runtime is not installed")
    lib = build_lib.build(sanitize=True,
                          out=str(tmp_path_factory.mktemp("san") / "libhga_san.so"))
    env = dict(os.environ, HGA_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return lib, rt, env


def test_sanitized_library_is_the_one_loaded(sanitized):
    lib, rt, env = sanitized
    code = ("import sparse_long_context_query_amd as h; h.lib(); "
            "print(open('/proc/self/maps').read())")
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    assert lib in r.stdout and os.path.realpath(rt) in r.stdout


def test_abi_checks_under_asan_ubsan(sanitized):
    _, _, env = sanitized
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-x", "-q", "-p", "no:cacheprovider"],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr

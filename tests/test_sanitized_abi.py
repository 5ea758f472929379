"""The C ABI checks of tests/test_abi.py, run against a build of the API
layer instrumented with AddressSanitizer and UndefinedBehaviorSanitizer on
the host (exact_range_similarity_amd/build.py, build_sanitized).  No GPU is
needed: every call there fails validation or finds no device before it
launches anything, which exercises the argument checks, the error paths and
the handle bookkeeping under the sanitizers."""
import os
import subprocess
import sys

import pytest

from exact_range_similarity_amd import build as ersj_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized():
    try:
        rt = ersj_build.sanitizer_runtime()
    except FileNotFoundError as e:
        pytest.skip(str(e))
    return ersj_build.build_sanitized(), rt


def test_sanitized_library_is_instrumented(sanitized):
    lib, _ = sanitized
    out = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report_load" in out or "__asan_load" in out
    assert "__ubsan_handle" in out


def test_abi_checks_pass_under_sanitizers(sanitized):
    lib, rt = sanitized
    env = dict(os.environ)
    env.update(ERSJ_LIBRARY=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout

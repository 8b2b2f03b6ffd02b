"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/abi_check.c (compiled as C, so the header is checked for C use too) sweeps
the size queries over boundary and extreme arguments and calls every entry point
with arguments it must reject; build.build_abi_check links it against the entry
points' host code rebuilt with both sanitizers on the host pass (any finding
aborts). Nothing here reaches a GPU."""
import os
import subprocess

import pytest

from subquadratic_sequence_amd import build as hybuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def abi_check():
    if not os.path.exists(os.path.join(ROOT, "subquadratic_sequence_amd", "libhyena.so")):
        pytest.skip("libhyena.so not built")
    return hybuild.build_abi_check()


def _run(exe):
    env = dict(os.environ)
    # the HIP runtime keeps process-lifetime allocations; leaks are not what is checked
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)


def test_sanitizers_are_linked(abi_check):
    out = subprocess.run(["nm", abi_check], capture_output=True, text=True, check=True).stdout
    assert "__asan_report_load" in out
    assert "__ubsan_handle_mul_overflow_abort" in out


def test_abi_validation_under_sanitizers(abi_check):
    r = _run(abi_check)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all expectations hold" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr

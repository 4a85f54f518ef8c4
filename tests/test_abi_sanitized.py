"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
tests/abi_check.cpp repeats the host-side argument checks of the ABI tests
(sizes, nulls, alignment, dtype, flags, composite blocks, the allocation-free
forward) in a program whose host code, api.cpp included, is built with both
sanitizers (device code as usual).  Any sanitizer report fails the run."""
import os
import shutil
import subprocess

import pytest

from linear_cross_entropy_cce_amd import build as BLD


def _have_hipcc():
    try:
        BLD.hipcc()
        return True
    except RuntimeError:
        return False


@pytest.mark.skipif(not _have_hipcc() or shutil.which("ld") is None, reason="needs hipcc")
def test_host_checks_under_sanitizers():
    exe = BLD.build_host_check()
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report
    assert "all host-side checks hold" in r.stdout, report
    assert "runtime error" not in report and "AddressSanitizer" not in report, report

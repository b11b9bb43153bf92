"""The ABI checks of tests/test_abi.py, run against the host-sanitizer build
of the library (favor_api.cpp compiled with AddressSanitizer and
UndefinedBehaviorSanitizer, any report fatal), in a child process that
preloads the sanitizer runtime.  Needs no GPU: every call in those tests
returns from the host checks or is a host-only function."""
import os
import subprocess
import sys

import pytest

from linear_kernelized_attention_amd import build as BLD

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hostsan_lib():
    if not os.path.exists(BLD.HOSTSAN_LIB):
        BLD.build_hostsan()
    return BLD.HOSTSAN_LIB


def test_hostsan_build_is_instrumented():
    out = subprocess.run(["nm", "-D", _hostsan_lib()], capture_output=True, text=True, check=True).stdout
    assert "__asan_report_load" in out and "__ubsan_handle" in out


def test_abi_checks_under_host_sanitizers():
    env = dict(os.environ)
    env.update(LD_PRELOAD=BLD.asan_runtime(), FAVOR_LIB=_hostsan_lib(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
    assert " passed" in tail, tail

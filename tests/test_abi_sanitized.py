"""The ABI validation tests again, against a build whose host side (mla_api.cpp)
is compiled with AddressSanitizer and UndefinedBehaviorSanitizer: an out-of-bounds
access, use after free, signed overflow or misaligned access anywhere in the
argument checks, ring/window arithmetic or workspace carving that the tests reach
aborts the run.  CPU only; no kernel is launched (MLA_FAULT_INJECT covers the
launch paths)."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, os.path.join(HERE, "sanitize"))


@pytest.fixture(scope="module")
def sanitized_lib():
    import build_host_sanitized as S
    if not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    return S.build(), S.asan_runtime()


def test_sanitized_build_is_instrumented(sanitized_lib):
    lib, _ = sanitized_lib
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle_" in syms


def test_abi_tests_pass_under_sanitizers(sanitized_lib):
    lib, runtime = sanitized_lib
    env = dict(os.environ, LD_PRELOAD=runtime, MLA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("MLA_FAULT_INJECT", None)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_abi_cpu.py"),
                        "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out

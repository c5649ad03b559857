"""The ABI tests (tests/test_abi.py) run against a host-only build of the
C-ABI layer instrumented with AddressSanitizer and UndefinedBehaviorSanitizer.

fa_api.cpp validates pointers, sizes and ranges with 64-bit arithmetic
before anything reaches the GPU; this run checks that arithmetic for
out-of-bounds accesses, overflow and other undefined behaviour. The kernel
launchers are stubs (tests/hostsan/stub_launch.cpp): every ABI test call is
stopped by validation before it would launch. The test builds the library
with g++, then runs the ABI tests in a child process that loads it first
after the ASan runtime, and fails on any sanitizer report.
"""

import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, os.path.join(HERE, "hostsan"))

import build_hostsan  # noqa: E402


needs_gxx = pytest.mark.skipif(
    build_hostsan.compiler() is None or build_hostsan.runtime_library() is None,
    reason="g++ with the ASan runtime is needed")


def sanitized_env(lib):
    env = dict(os.environ)
    env["FA_LIBRARY"] = lib
    preload = [build_hostsan.runtime_library()] + [p for p in env.get("LD_PRELOAD", "").split(":")
                                                   if p]
    env["LD_PRELOAD"] = ":".join(preload)
    # The interpreter and torch are not instrumented: leak checking at exit
    # would report their allocations, so only memory errors and UB count.
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


@needs_gxx
def test_abi_suite_under_host_sanitizers():
    lib = build_hostsan.build()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_handle" in syms  # instrumented
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_abi.py"),
                          "-q", "-p", "no:cacheprovider", "-x"],
                         cwd=ROOT, env=sanitized_env(lib), capture_output=True, text=True,
                         timeout=600)
    out = res.stdout + res.stderr
    print(out[-3000:])
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert res.returncode == 0, out[-3000:]
    assert " passed" in out


def test_abi_tests_load_the_library_they_are_given():
    """FA_LIBRARY selects the build the ABI tests load (the sanitized one
    above); without it the in-tree libfa.so is used."""
    code = ("import exact_attention_120_amd._lib as L; print(L.LIB_PATH)")
    env = dict(os.environ, FA_LIBRARY="/nonexistent/libfa_other.so")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=300)
    assert res.stdout.strip() == "/nonexistent/libfa_other.so", res.stderr


@needs_gxx
@pytest.mark.parametrize("call,reports", [
    # UBSan's object-size check or ASan's shadow check, whichever fires first
    ("planted_heap_overflow(4)", ("heap-buffer-overflow", "insufficient space for an object")),
    ("planted_signed_overflow(5)", ("signed integer overflow",))])
def test_sanitized_run_reports_planted_mistakes(call, reports):
    """The same flags and loading catch a heap overflow and a signed
    overflow planted in a host library of their own."""
    lib = build_hostsan.build_planted()
    code = f"import ctypes; ctypes.CDLL({lib!r}).{call}"
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=sanitized_env(lib),
                         capture_output=True, text=True, timeout=120)
    assert res.returncode != 0 and any(r in res.stderr for r in reports), res.stderr[-2000:]

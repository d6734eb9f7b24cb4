"""The C-ABI host layer under AddressSanitizer and UBSan: argument
validation, dispatch, workspace carving and the error string.

libffd_san.so is the same library with both sanitizers on the host pass of
ffd_api.hip and ffd_quantize.hip (device code is not instrumented).
tests/test_abi.py runs against it in a child Python with the ASan runtime
preloaded (FFD_LIBRARY selects the build). Any report fails the run.
No GPU is used."""

import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_long_context_ffd_amd")


def _build():
    sys.path.insert(0, PKG)
    try:
        import build
    finally:
        sys.path.remove(PKG)
    return build, build.build_sanitized()


def test_abi_tests_clean_under_asan_and_ubsan():
    build, lib = _build()
    rt = build.asan_runtime()
    assert os.path.exists(rt), rt
    undef = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in undef and "__ubsan_handle" in undef, "library is not instrumented"
    env = dict(os.environ, LD_PRELOAD=rt, FFD_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the child maps the sanitized build, not libffd.so
    probe = subprocess.run(
        [sys.executable, "-c",
         "import sparse_long_context_ffd_amd as f; f.lib(); print(open('/proc/self/maps').read())"],
        env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-2000:]
    maps = probe.stdout
    assert "libffd_san.so" in maps and not re.search(r"/libffd\.so\b", maps)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-m", "not gpu", "-p", "no:cacheprovider"],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert re.search(r"\b\d+ passed\b", out), out[-2000:]

"""The host code of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

capi.cpp is built host-only with both sanitizers (tests/c/build_sanitized.py)
and every C-ABI validation case of tests/test_abi_cpu.py runs against that
build in a child process with the sanitizer runtime preloaded: fake device
pointers, overflowing sizes, misaligned and overlapping buffers, grids past
the 32-bit limit.  Any report aborts the child (no recovery), so the cases
must pass with a clean exit.  No device work is started.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = """
import sys
sys.path.insert(0, {root!r})
import sequence_dit_attention_amd._lib as L
L.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", {tests!r}]))
"""


def test_abi_validation_cases_under_asan_and_ubsan():
    from tests.c import build_sanitized

    lib = build_sanitized.build()
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the library is not instrumented"
    env = dict(os.environ)
    env["LD_PRELOAD"] = build_sanitized.runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = CHILD.format(root=ROOT, lib=lib, tests=os.path.join(ROOT, "tests", "test_abi_cpu.py"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]

"""The library's host-side argument checks under AddressSanitizer and UndefinedBehaviorSanitizer.
tests/c_abi/validate.c calls every entry point with invalid and empty arguments, and with byte
extents past the library's limit (134 calls),
against a build whose host code is instrumented: every status must match what the header
documents, and neither sanitizer may report. Host code only; no GPU is needed."""
import importlib.util
import os
import shutil
import subprocess

import pytest

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi")


def test_argument_validation_under_sanitizers():
    script = os.path.join(HERE, "build_sanitized.py")
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")) or not os.path.exists(script):
        pytest.skip("hipcc or the sanitizer build script is not available")
    spec = importlib.util.spec_from_file_location("kvx_build_sanitized", script)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    exe = mod.build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "validated 134 calls, 0 mismatches" in r.stdout, r.stdout
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr

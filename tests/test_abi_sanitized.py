"""The C-ABI host code under AddressSanitizer and UndefinedBehaviorSanitizer:
the CPU ABI tests (argument validation, size and overlap arithmetic,
workspace sizing; no kernel launch) rerun against a build of api.cpp with
both sanitizers, in a subprocess that preloads the ASan runtime.  Any
sanitizer report aborts that process and fails this test."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_host_sanitizers():
    from exact_attention_69_amd import build as b
    runtime = b.asan_runtime()
    if runtime is None:
        pytest.skip("clang's shared ASan runtime is not installed")
    lib = b.build_sanitized()
    env = dict(os.environ, EXATTN_LIBRARY=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:detect_odr_violation=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x",
                          "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]

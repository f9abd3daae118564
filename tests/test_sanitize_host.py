"""The C-ABI library's CPU tests (tests/test_abi.py: argument validation,
work division, workspace sizes, error reporting; no GPU work) rerun against
a build of the host code with AddressSanitizer and
UndefinedBehaviorSanitizer (csrc/build_sanitize.py). Any sanitizer report
fails the run (undefined behaviour aborts; -s keeps the reports in the
captured output)."""

import os
import subprocess
import sys

import pytest

from tests.conftest import ROOT

CSRC = os.path.join(ROOT, "compressed_decode_attention_quantize_amd", "csrc")


@pytest.mark.timeout(900)
def test_abi_tests_under_asan_ubsan():
    sys.path.insert(0, CSRC)
    try:
        import build_sanitize as bs
    finally:
        sys.path.pop(0)
    if not os.path.exists(bs.CLANGXX):
        pytest.skip("no ROCm clang++")
    try:
        runtime = bs.asan_runtime()
    except FileNotFoundError as e:
        pytest.skip(str(e))
    lib = bs.build_sanitized()
    env = dict(os.environ, TQ_LIBRARY=lib, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0")
    res = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "-q", "-x", "-s", "-p", "no:cacheprovider"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]

"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds libnomas with the host side instrumented (address and undefined-behaviour
sanitizers, no recovery; device code as usual) and runs the C-ABI checks of test_abi.py
against it in a child process with the ASan runtime preloaded: every argument
check, size plan and descriptor update those tests reach runs instrumented, and
any out-of-bounds access, use after free or undefined behaviour ends the child
with a report. No GPU is needed (those calls return before any launch)."""

import os
import subprocess
import sys

import pytest

from segment_autoregressive_dit_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
from segment_autoregressive_dit_amd import nomas
nomas.LIB_PATH = {lib!r}
import pytest
rc = pytest.main(["-q", "-p", "no:cacheprovider", {abi!r}])
maps = open("/proc/self/maps").read()
assert {lib!r} in maps, "the instrumented library was not the one loaded"
assert "libclang_rt.asan" in maps, "the ASan runtime is not loaded"
sys.exit(int(rc))
"""


def test_abi_checks_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(B.ASAN_RUNTIME):
        pytest.skip("no ASan runtime in this toolchain")
    lib = str(tmp_path / "libnomas_sanitized.so")
    B.build(verbose=False, sanitize=True, out=lib)
    env = dict(os.environ, LD_PRELOAD=os.path.realpath(B.ASAN_RUNTIME),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib,
                        abi=os.path.join(ROOT, "tests", "test_abi.py"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    report = r.stdout[-4000:] + r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in report and "runtime error:" not in report, report
    assert r.returncode == 0, report
    assert "passed" in r.stdout, report

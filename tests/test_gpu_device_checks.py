"""The GPU parity tests of the RoPE, cache, frame-range, fused-projection,
block-causal and sparse paths run against the checking build (libnomas_debug.so: every
cache slot, token range and tile row a kernel addresses is tested against its
buffer, failures counted on the device and the access skipped). They must pass
as they do on the normal build, with no failed check.

Runs in a child process so that the checking library is the one loaded there;
the child asserts that it is mapped and reads the device's failure count after
the tests."""

import os
import subprocess
import sys

import pytest

from segment_autoregressive_dit_amd import build as B

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
sys.path.insert(0, {tests!r})
from segment_autoregressive_dit_amd import nomas
nomas.LIB_PATH = {lib!r}
import pytest
rc = pytest.main(["-q", "-x", "-p", "no:cacheprovider", "-m", "gpu"] + {args!r})
maps = open("/proc/self/maps").read()
assert {lib!r} in maps, "the checking library was not the one loaded"
n = nomas.nomas_device_check_failures(True)
print(f"device check failures: {{n}}", flush=True)
sys.exit(int(rc) if rc else (0 if n == 0 else 3))
"""


def test_parity_tests_pass_on_the_checking_build_with_no_failed_check():
    assert os.path.exists(B.DEBUG_LIB), "libnomas_debug.so is missing (build() builds it)"
    t = os.path.join(ROOT, "tests")
    args = [os.path.join(t, "test_gpu_rope.py"), os.path.join(t, "test_gpu_kvcache.py"),
            os.path.join(t, "test_gpu_frames.py"),
            os.path.join(t, "test_gpu_pipeline.py"), os.path.join(t, "test_gpu_block_causal.py"),
            os.path.join(t, "test_gpu_sparse.py"),
            os.path.join(t, "test_gpu_qkv.py") + "::test_projection_append_equals_projection_then_append",
            os.path.join(t, "test_gpu_qkv.py") + "::test_projection_vt_is_the_value_channels_transposed",
            os.path.join(t, "test_gpu_fuzz.py"), "-k", "not medium"]
    code = CHILD.format(root=ROOT, tests=t, lib=B.DEBUG_LIB, args=args)
    r = subprocess.run([sys.executable, "-u", "-c", code], capture_output=True, text=True, timeout=900)
    report = r.stdout[-4000:] + r.stderr[-2000:]
    assert "device check failures: 0" in r.stdout, report
    assert r.returncode == 0, report

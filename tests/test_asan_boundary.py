"""The host-side boundary tests run again against a build of the library whose host code is
compiled with AddressSanitizer (its runtime preloaded into a child Python), so argument
validation, size queries and status strings are checked for out-of-bounds accesses and
use-after-free on the CPU, without a GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_boundary_tests_pass_under_host_asan():
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import asan_build

    rt = asan_build.runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime next to hipcc")
    lib = asan_build.build()
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    env["LWM_ATTN_LIBRARY"] = lib
    # leak checking would report the Python interpreter's own allocations
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=86"
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_boundary.py"), "-k", "not wrappers_check_buffer_sizes"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out

"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library's sources are rebuilt with the host side instrumented (the device
side is compiled but never runs), and the C-ABI tests that need no GPU -- the
argument checks of every entry point, the layer predicate, the binding's checks
-- run against that build in a child process that preloads the sanitizer
runtime.  Any report (heap or stack overflow, use after free, signed overflow,
misaligned or null access, invalid shift) aborts the child and fails this test.
Runs only where no GPU is present: the ABI tests pass fake device pointers that
only a machine without a gfx950 is sure to reject before a launch.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(os.path.exists("/dev/kfd"),
                                reason="host-only check: runs where no GPU is present")


def test_abi_checks_under_host_sanitizers(tmp_path):
    from nvfp4_block_scaled_05_amd import build
    lib = build.build_host_sanitized(str(tmp_path / "sanitize"))
    env = dict(os.environ)
    env.update({
        "NVFP4_LIBRARY": lib,
        "LD_PRELOAD": build.asan_runtime(),
        # Python and the HIP runtime are not instrumented and keep allocations
        # for the life of the process: leak reports would be theirs
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
        "PYTHONDONTWRITEBYTECODE": "1",
    })
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
           "tests/test_abi.py", "tests/test_binding_checks.py", "tests/test_oracle_layers.py"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
    # the child really loaded the sanitizer build
    check = [sys.executable, "-c",
             "from nvfp4_block_scaled_05_amd import _binding; print(_binding.LIB_PATH)"]
    r2 = subprocess.run(check, cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r2.stdout.strip() == lib, r2.stdout + r2.stderr

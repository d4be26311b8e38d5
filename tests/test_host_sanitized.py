"""The host tests again, against the host-only sanitizer build of libspb
(spb_host.cpp under AddressSanitizer and UndefinedBehaviorSanitizer): the
planner, the plan accessors and every host-side validation run with bounds,
use-after-free and undefined-behaviour checks, in a child process started with
the ASan runtime preloaded.  No GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_TESTS = ["tests/test_host_plan.py", "tests/test_host_templates.py", "tests/test_host_layer.py"]

CHILD = r"""
import sys
import shared_prefix_branch_amd as spb
spb.lib()
maps = open("/proc/self/maps").read()
assert "libspb_host_san.so" in maps and "libasan" in maps, "the sanitizer build is not the loaded library"
import pytest
sys.exit(pytest.main(["-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider"] + sys.argv[1:]))
"""


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_host_tests_under_address_and_ub_sanitizers():
    from shared_prefix_branch_amd import build as B
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = B.SAN_LIB if os.path.exists(B.SAN_LIB) else B.build_host_sanitized()
    env = dict(os.environ, LD_PRELOAD=asan, SPB_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", CHILD] + HOST_TESTS, cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert " passed" in out, out[-2000:]

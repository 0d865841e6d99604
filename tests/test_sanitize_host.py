"""The C-ABI layer (argument checks, workspace layouts, launch sequencing in
gdn_api.hip) under host-only AddressSanitizer and UndefinedBehaviorSanitizer:
a build of libgdn.so whose host code is instrumented runs the ABI tests
(tests/test_abi.py, every entry point and every refusal path, nothing
launched) in a fresh process with the ASan runtime preloaded. Any memory
error or undefined behaviour aborts that process. CPU only."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

RUNNER = r"""
import sys
sys.path.insert(0, {root!r})
from frame_wise_gated_amd import gdn
gdn.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main([{tests!r}, "-q", "-m", "not gpu", "-p", "no:cacheprovider"]))
"""


def test_abi_tests_pass_under_host_asan_and_ubsan(tmp_path):
    from frame_wise_gated_amd import build

    try:
        lib = build.build_sanitized(str(tmp_path))
        rt = build.sanitizer_runtime()
    except (RuntimeError, subprocess.CalledProcessError, FileNotFoundError) as e:
        pytest.fail(f"sanitized build failed: {e}")
    assert os.path.exists(rt), rt
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = RUNNER.format(root=ROOT, lib=lib, tests=os.path.join(ROOT, "tests", "test_abi.py"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in r.stdout
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]

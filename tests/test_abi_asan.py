"""The CPU tests of the C ABI (tests/test_abi.py) again, against a build of the library whose host
code is instrumented with AddressSanitizer (argument validation, workspace sizing and the error
text run under the sanitizer; no GPU is needed, nothing is launched)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_suite_under_host_asan():
    from causal_sliding_window_attn_amd import build

    try:
        lib = build.build_asan()
        rt = build.asan_runtime()
    except RuntimeError as e:  # no HIP toolchain on this host
        pytest.skip(str(e))
    env = dict(os.environ, SWATTN_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "AddressSanitizer" not in r.stderr, r.stderr[-3000:]

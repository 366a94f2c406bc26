"""The C ABI's host-side argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, no kernel is launched).

The library is rebuilt with the host sanitizers (build.build_host_sanitized,
into the test's temporary directory) and the host ABI and binding tests run against it in a child process that
preloads the compiler's AddressSanitizer runtime; any report aborts that
process. The validated domains are those of page "Configurable H100
consistency runs", sampling paragraph (per-row parameters) and the layout of
its topology paragraph (padded vocabulary, canonical shards).
"""
import os
import subprocess
import sys

import pytest

from invariant_token_log_fp32_amd import build

pytestmark = pytest.mark.slow


def test_host_validation_is_clean_under_asan_and_ubsan(tmp_path):
    runtime = build.asan_runtime()
    if not runtime:
        pytest.skip("the compiler's AddressSanitizer runtime was not found")
    lib = build.build_host_sanitized(str(tmp_path / "librlk_logp_hostsan.so"))
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True)
    if nm.returncode == 0:  # the host code carries the sanitizers' checks
        assert "__asan_report" in nm.stdout and "__ubsan_handle" in nm.stdout
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ)
    env.update({
        "RLK_LIBRARY": lib,
        "LD_PRELOAD": runtime,
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          "tests/test_abi_host.py", "tests/test_binding_host.py"],
                         cwd=root, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out

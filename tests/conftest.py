import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session", autouse=True)
def _library_built():
    """Build librlk_logp.so when it is missing (a fresh checkout)."""
    from invariant_token_log_fp32_amd import LIB_PATH
    if not os.path.exists(LIB_PATH):
        from invariant_token_log_fp32_amd import build
        build.build()


def pytest_terminal_summary(terminalreporter):
    gpu_util = sys.modules.get("gpu_util")
    if gpu_util is not None and gpu_util.REPORT:
        terminalreporter.write_sep("-", "counts reported by the GPU tests")
        for line in gpu_util.REPORT:
            terminalreporter.write_line(line)

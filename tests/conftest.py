import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library through its C ABI")
    if os.environ.get("RMSQ_SANITIZE") == "1":
        # tests/sanitize/run_sanitized.py: the oracle and the library's host
        # layer built under ASan / UBSan (their runtimes preloaded)
        import fp4_activation_quantization_amd as rq
        import oracle

        san = os.path.join(ROOT, "tests", "sanitize")
        rq.LIB_PATH = os.path.join(san, "librmsq.so")
        oracle.LIB_PATH = os.path.join(san, "liboracle.so")
        for p in (rq.LIB_PATH, oracle.LIB_PATH):
            if not os.path.exists(p):
                raise pytest.UsageError(f"{p} is missing: run tests/sanitize/run_sanitized.py")
        if "libasan" not in os.environ.get("LD_PRELOAD", ""):
            raise pytest.UsageError("RMSQ_SANITIZE=1 needs the sanitizer runtimes preloaded (run_sanitized.py)")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    return oracle.lib()

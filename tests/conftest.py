import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle

    return oracle.load()


@pytest.fixture(autouse=True)
def _default_plan_rule():
    """Every test starts and ends on the default plan rule (tests that force a
    plan set the library's override themselves)."""
    from dense_fp16_gemm_03_amd import gemm

    def reset():
        if gemm._lib is not None or os.path.exists(gemm.LIBRARY):
            gemm.gemm_f16_set_plan_override("")

    reset()
    yield
    reset()

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _has_gpu() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    if not _has_gpu():
        pytest.skip("no GPU visible")
    import torch
    from block_diffusion_draft_vocab_amd import ddt
    ddt.load()            # raises loudly if the HIP library is missing
    return torch.device("cuda:0")


def pytest_sessionfinish(session, exitstatus):
    """Write the largest errors the parity tests measured (tests/report.py)
    to the JSON file named by DDT_PARITY_REPORT, when that is set."""
    path = os.environ.get("DDT_PARITY_REPORT")
    if not path:
        return
    from tests import report
    if report.ERRORS:
        report.dump(path)

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running")


@pytest.fixture(scope="session")
def has_gpu():
    import torch
    return torch.cuda.is_available()


@pytest.fixture(params=["persistent", "per_op"])
def decode_path(request):
    """Runs the test once per decode path: the persistent kernel (default) and the per-op
    kernels (RIVER_PERSIST=0 at context creation)."""
    old = os.environ.get("RIVER_PERSIST")
    os.environ["RIVER_PERSIST"] = "1" if request.param == "persistent" else "0"
    yield request.param
    if old is None:
        del os.environ["RIVER_PERSIST"]
    else:
        os.environ["RIVER_PERSIST"] = old


_NEAR = {"checked": 0, "near": 0}


@pytest.fixture(autouse=True)
def near_tie_budget():
    """Counts the greedy-token comparisons a test makes (tests/_util.top1_checked). A test fails
    when more than max(2, MAX_NEAR_TIE_FRAC of them) were near ties (not compared: greedy decoding
    of a random-weight model often repeats a token, so one near tie can recur on the next
    steps); the session's totals are reported at the end and bounded by the same fraction."""
    from tests import _util
    _util.TOP1["checked"] = _util.TOP1["near"] = 0
    yield
    n, near = _util.TOP1["checked"], _util.TOP1["near"]
    _NEAR["checked"] += n
    _NEAR["near"] += near
    if n:
        print(f"top-1 comparisons: {n}, near ties (not compared): {near}")
    assert near <= max(2, int(_util.MAX_NEAR_TIE_FRAC * n)), f"{near} near-tied steps of {n}"


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    if _NEAR["checked"]:
        terminalreporter.write_line(f"greedy top-1 comparisons: {_NEAR['checked']}, near ties not "
                                    f"compared: {_NEAR['near']}")


def pytest_sessionfinish(session, exitstatus):
    from tests import _util
    if _NEAR["checked"] >= 20 and _NEAR["near"] > _util.MAX_NEAR_TIE_FRAC * _NEAR["checked"]:
        session.exitstatus = 1

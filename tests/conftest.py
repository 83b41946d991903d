import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workloads")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def ts():
    """The HIP library binding; GPU tests fail loudly if it cannot load."""
    if not gpu_available():
        pytest.skip("no GPU visible")
    from convolution_voxelised_point_amd import ts as _ts
    return _ts


def pytest_terminal_summary(terminalreporter):
    """Error distribution of every feature comparison the session made."""
    helpers = sys.modules.get("helpers")
    log = getattr(helpers, "PARITY_LOG", None)
    if not log:
        return
    tr = terminalreporter
    tr.section("feature parity: |GPU - fp64 oracle| per comparison")
    tr.write_line(f"{'comparison':58s} {'elements':>10s} {'max|ref|':>10s} {'p50':>10s} {'p99':>10s} "
                  f"{'max':>10s} {'max/max|ref|':>12s}  bar")
    for what, n, m, p50, p99, mx, rel, bar in log:
        tr.write_line(f"{what[:58]:58s} {n:10d} {m:10.3e} {p50:10.3e} {p99:10.3e} {mx:10.3e} {rel:12.3e}  {bar}")

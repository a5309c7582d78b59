import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Worst decode errors per parity case (relative row error against the
    2e-3 bar; absolute lse difference and the largest share of its bar, the
    bar including the fp32 slack of large-magnitude cases), printed even
    with -q."""
    try:
        from harness import PARITY_LOG
    except Exception:
        return
    if not PARITY_LOG:
        return
    tr = terminalreporter
    tr.write_sep("-", "decode parity margins (bars: row rel err <= 2e-3; |d lse| <= 2e-3 + fp32 slack)")
    for case, rel, dl, rows, use in PARITY_LOG:
        tr.write_line(f"{case:<40s} rows {rows:5d}  worst rel {rel:.2e} ({rel / 2e-3:4.0%} of bar)  "
                      f"worst |d lse| {dl:.2e} ({use:4.0%} of its bar)")

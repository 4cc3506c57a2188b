import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU case")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    import oracle
    oracle.build()
    yield


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """One line per parity kind: how many cases were compared and the worst
    margin, so that the numbers survive a quiet (-q) run."""
    mod = sys.modules.get("gpu_util")
    rows = getattr(mod, "RESULTS", None) if mod else None
    if not rows:
        return
    kinds = {}
    for r in rows:
        kinds.setdefault(r["kind"], []).append(r)
    for kind, rs in sorted(kinds.items()):
        if "max_err" in rs[0]:
            worst = max(rs, key=lambda r: r["max_err"] / r["bound"])
            terminalreporter.write_line(
                f"parity[{kind}]: {len(rs)} cases, worst max|err| {worst['max_err']:.3e} "
                f"(bound {worst['bound']:.0e}) in {worst['case']}; worst lse err "
                f"{max(r.get('lse_err', 0.0) for r in rs):.3e}")
        else:
            terminalreporter.write_line(f"parity[{kind}]: {len(rs)} cases, all exact")

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: large oracle or GPU workloads")


GOLDEN = os.path.join(ROOT, "tests", "golden")


@pytest.fixture(scope="session")
def golden_dir():
    return GOLDEN


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Parity margins of the GPU tests that ran: the worst checks (max error
    over tolerance), and every check as JSON in the file $RA_PARITY_JSON
    names, when it is set."""
    import json
    helpers = sys.modules.get("tests.gpu_helpers")
    rows = list(getattr(helpers, "MARGINS", []) or [])
    if not rows:
        return
    for r in rows:
        r["ratio"] = r["err"] / r["tol"] if r["tol"] > 0 else float("inf")
    rows.sort(key=lambda r: -r["ratio"])
    tr = terminalreporter
    tr.section("parity margins: max error / tolerance (worst first)")
    for r in rows[:12]:
        tr.write_line(f"{r['ratio']:.3f}  {r['name']}  err={r['err']:.2e} tol={r['tol']:.0e}")
    tr.write_line(f"{len(rows)} parity checks recorded; worst ratio {rows[0]['ratio']:.3f}")
    out = os.environ.get("RA_PARITY_JSON")
    if out:
        with open(out, "w") as f:
            json.dump(rows, f, indent=1)

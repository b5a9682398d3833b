import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def pytest_terminal_summary(terminalreporter):
    """Parity record of the session: every comparison against the fp64 oracle, with the
    elements that passed only as rounding-limited (allowed in named short-context cases)."""
    mod = sys.modules.get("gpu_util")
    recs = getattr(mod, "RECORDS", None)
    if not recs:
        return
    tr = terminalreporter
    n = sum(r["n"] for r in recs)
    rl = sum(r["rounding_limited"] for r in recs)
    strict = [r for r in recs if not r["relief"]]
    tr.write_sep("-", "parity against the fp64 oracle (|err| <= 2e-3 + 2e-3 |ref|)")
    tr.write_line(f"comparisons {len(recs)} ({len(strict)} strict), elements {n}, "
                  f"rounding-limited {rl}, max abs err {max(r['max_abs'] for r in recs):.3e}")
    for r in recs:
        if r["rounding_limited"]:
            tr.write_line(f"  rounding-limited {r['rounding_limited']} of {r['n']} "
                          f"(format cannot meet the bound at {r['unattainable']}): "
                          f"{r['test']} {r['label']}")
    full = [r for r in recs if "full_size" in r["test"]]
    if full:
        tr.write_line(f"full-size comparisons {len(full)}, elements "
                      f"{sum(r['n'] for r in full)}, rounding-limited "
                      f"{sum(r['rounding_limited'] for r in full)}, worst abs err "
                      f"{max(r['max_abs'] for r in full):.3e}")

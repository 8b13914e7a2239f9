import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Worst parity margin per test file: the largest |gpu - oracle| / tolerance
    over every element checked (1.0 is the bar), with its case, and the largest
    absolute and relative errors seen in that file."""
    try:
        from helpers import MARGINS
    except ImportError:
        return
    if not MARGINS:
        return
    per_file = {}
    for test, what, max_abs, max_rel, ratio in MARGINS:
        f = test.split("::")[0]
        d = per_file.setdefault(f, {"n": 0, "ratio": -1.0, "case": "", "abs": 0.0, "rel": 0.0})
        d["n"] += 1
        d["abs"] = max(d["abs"], max_abs)
        d["rel"] = max(d["rel"], max_rel)
        if ratio > d["ratio"]:
            d["ratio"], d["case"] = ratio, f"{test} [{what}]"
    tr = terminalreporter
    tr.write_sep("-", "parity margins against the oracle (bar: err/tol <= 1)")
    for f, d in sorted(per_file.items()):
        tr.write_line(f"{f}: {d['n']} checks, worst err/tol {d['ratio']:.3f}, "
                      f"max_abs {d['abs']:.3e}, max_rel {d['rel']:.3e}; worst case {d['case']}")

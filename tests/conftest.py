import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; calls the HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests fail loudly (not skip) when run on a machine without a GPU and
    # selected explicitly; when deselected with -m "not gpu" they never run.
    pass


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Floating-point parity report: for each compared quantity, the worst
    per-row relative L2 error and the worst element error relative to its
    scale (max(|ref|, row rms), or a Cauchy-Schwarz bound), each to be read
    against the tolerance, seen in this session."""
    mod = sys.modules.get("gpu_util")
    rep = getattr(mod, "REPORT", None) if mod is not None else None
    if not rep:
        return
    out = os.environ.get("PARITY_REPORT")
    if out:
        import json
        with open(out, "w") as f:
            json.dump(rep, f, indent=1)
    agg = {}
    for r in rep:
        key = r["test"].split("::")[0].replace("tests/", "") + " " + r["what"].split(" ")[0]
        a = agg.setdefault(key, dict(n=0, rows=0, row=0.0, elem=0.0, tol=r["tol"]))
        a["n"] += 1
        a["rows"] += r["rows"]
        if r["worst_row_l2"] == r["worst_row_l2"]:
            a["row"] = max(a["row"], r["worst_row_l2"])
        a["elem"] = max(a["elem"], r["worst_elem_rel"])
        a["tol"] = max(a["tol"], r["tol"])
    terminalreporter.write_sep("-", f"FP parity: {len(rep)} checks (worst per quantity)")
    terminalreporter.write_line(f"{'file quantity':58s} {'checks':>6s} {'rows':>9s} "
                                f"{'row L2':>9s} {'elem':>9s} {'tol':>7s}")
    for k in sorted(agg):
        a = agg[k]
        terminalreporter.write_line(f"{k[:58]:58s} {a['n']:6d} {a['rows']:9d} {a['row']:9.2e} "
                                    f"{a['elem']:9.2e} {a['tol']:7.0e}")

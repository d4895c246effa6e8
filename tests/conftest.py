import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
    # GPU tests run on a GPU machine only; on a CPU-only host they are skipped with a reason.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


# ---- parity report: one machine-readable record of a session that ran GPU
# tests (each test's outcome and duration, the comparison rules, the accepted
# near-ties), written to OCRDEC_PARITY_REPORT (default
# gpurun_out/parity_report.json).
_RESULTS = []


def pytest_runtest_logreport(report):
    if report.when == "call" or (report.when == "setup" and report.outcome != "passed"):
        _RESULTS.append({"test": report.nodeid, "outcome": report.outcome, "seconds": round(report.duration, 3),
                         "gpu": "gpu" in report.keywords})


def pytest_sessionfinish(session, exitstatus):
    ran_gpu = [r for r in _RESULTS if r["gpu"] and r["outcome"] != "skipped"]
    if not ran_gpu:
        return
    import json
    try:
        from tests import gpu_util as G
        rules = {"rel_tol": G.REL_TOL, "flip_fraction": G.FLIP_FRACTION, "near_tie": G.NEAR_TIE}
        ties = list(G.NEAR_TIES)
    except Exception:
        rules, ties = {}, []
    counts = {}
    for r in _RESULTS:
        counts[r["outcome"]] = counts.get(r["outcome"], 0) + 1
    rep = {"exit_status": int(exitstatus), "counts": counts, "rules": rules, "near_ties": ties, "tests": _RESULTS}
    path = os.environ.get("OCRDEC_PARITY_REPORT", os.path.join("gpurun_out", "parity_report.json"))
    try:
        os.makedirs(os.path.dirname(path) or ".", exist_ok=True)
        with open(path, "w") as f:
            json.dump(rep, f, indent=1)
    except OSError:
        pass

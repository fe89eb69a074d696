import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Totals of the GPU/oracle verification comparisons: requests compared, and the
    near-threshold cases (accept flags within 1e-6 of p(x)/q(x), tokens within 1e-6 R of a
    CDF boundary) that the parity contract counts instead of comparing bit for bit."""
    try:
        import parity
    except Exception:  # pragma: no cover
        return
    reps = parity.REPORTS
    if not reps:
        return
    tot = {k: sum(r[k] for r in reps) for k in ("requests", "accept_tests", "near_accept", "near_token",
                                                 "token_equal")}
    terminalreporter.write_line(
        f"verification parity: {len(reps)} comparisons, {tot['requests']} requests, {tot['accept_tests']} accept "
        f"tests; near_accept {tot['near_accept']}, near_token {tot['near_token']}, tokens equal {tot['token_equal']}")
    for r in reps:
        if r["near_accept"] or r["near_token"]:
            terminalreporter.write_line(f"  {r['label'] or '?'}: requests {r['requests']}, near_accept "
                                        f"{r['near_accept']}, near_token {r['near_token']}")

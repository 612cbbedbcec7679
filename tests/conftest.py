import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped (not failed) when no GPU is visible, so that a
    # plain `pytest tests/` on a CPU host stays green; `-m gpu` on a GPU machine
    # runs them for real.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    # max|dO| / max|V| of the comparisons run in this session: every case held
    # to a derived bound above the contract's 1e-2, and the worst of the rest
    try:
        from helpers import MARGINS, O_TOL
    except ImportError:  # pragma: no cover
        return
    if not MARGINS:
        return
    tr = terminalreporter
    tr.section("parity margins: max|dO| / max|V|")
    loose = [m for m in MARGINS if m[2] > O_TOL]
    strict = [m for m in MARGINS if m[2] <= O_TOL]
    for case, ratio, bar in loose:
        tr.write_line(f"{ratio:.3e} (bar {bar}) {case}")
    if strict:
        case, ratio, bar = max(strict, key=lambda m: m[1])
        tr.write_line(f"{len(strict)} comparisons at bar {O_TOL}: worst {ratio:.3e} ({case})")

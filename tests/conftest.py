import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_available() -> bool:
    try:
        import torch
        return bool(torch.cuda.is_available())
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible in this process (GPU tests run on the MI355X box)")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """The literal figure max|err| / rms(y_oracle) of every full-size workload
    compared in this run (and, for bf16 outputs, the figure the tests bound:
    max(|err| - 2^-8 |y|) / rms), so it can be read beside the 2e-2 bar."""
    try:
        from tests.gpu_util import LITERAL
    except Exception:
        return
    rows = sorted((w, v) for w, v in LITERAL.items() if w.startswith("config"))
    if not rows:
        return
    tr = terminalreporter
    tr.write_sep("-", "max|err|/rms per full-size workload (bar 2e-2)")
    for w, (lit, r15) in rows:
        extra = "" if r15 is None else f"   max(|err|-2^-8|y|)/rms {r15:.3e}"
        tr.write_line(f"{w:48s} max|err|/rms {lit:.3e}{extra}")

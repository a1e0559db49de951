import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU-oracle case")


def pytest_terminal_summary(terminalreporter):
    """Argmax parity of every lm_head check that ran: rows where the GPU and
    the oracle legitimately disagree (an FP16 rounding boundary within the
    FP32 accumulation error), shown even under -q."""
    gu = sys.modules.get("gpu_util")
    recs = getattr(gu, "ARGMAX_RECORDS", None) if gu else None
    if not recs:
        return
    amb = sum(r[1] for r in recs)
    rows = sum(r[2] for r in recs)
    terminalreporter.write_sep("-", f"argmax parity: {len(recs)} checks, {rows} rows, {amb} ambiguous")
    for what, a, n in recs:
        if a:
            terminalreporter.write_line(f"  {what}: {a} of {n} rows ambiguous")

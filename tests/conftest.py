import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Totals of every GPU-vs-oracle comparison of the session: how many
    output elements were judged, how many by the one-ulp bound for
    |O_ref| >= 2 (and how close they came), the worst |err|, cosine and lse
    error."""
    try:
        import attn_compare
    except ImportError:
        return
    recs = attn_compare.RECORDS
    if not recs:
        return
    n = sum(r[1] for r in recs)
    n_ulp = sum(r[2] for r in recs)
    worst_ulp = max(r[3] for r in recs)
    tr = terminalreporter
    tr.write_sep("-", "GPU-vs-oracle parity totals")
    tr.write_line(f"{len(recs)} comparisons, {n} output elements; {n_ulp} elements with |O_ref| >= 2 judged by the "
                  f"one-ulp bound (worst {worst_ulp:.3f} ulp; {sum(1 for r in recs if r[2])} comparisons had any)")
    tr.write_line(f"max |err| {max(r[4] for r in recs):.3e}, min cosine {min(r[5] for r in recs):.7f}, "
                  f"max lse err {max(r[6] for r in recs):.3e}")

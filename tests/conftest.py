import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_available():
    import torch
    return torch.cuda.is_available()


def pytest_terminal_summary(terminalreporter):
    """Summary of the parity comparisons: per dtype, the largest raw output error, the total
    count of elements beyond the literal tolerance, and the largest LSE error."""
    try:
        import parity_log
    except ImportError:
        return
    recs = parity_log.RECORDS
    if not recs:
        return
    tr = terminalreporter
    tr.section("parity against the fp64 oracle (raw errors)")
    for dt in sorted({r["dtype"] for r in recs}):
        rs = [r for r in recs if r["dtype"] == dt]
        worst = max(rs, key=lambda r: r["max_abs"])
        tr.write_line(
            f"{dt}: {len(rs)} comparisons, {sum(r['elements'] for r in rs)} elements; "
            f"max-abs {worst['max_abs']:.3e} ({worst['where']}); elements beyond the literal "
            f"tolerance {sum(r['beyond_tol'] for r in rs)}; lse max-abs "
            f"{max(r['lse_max_abs'] for r in rs):.3e}")
    for r in recs:
        if r["literal_gate"]:
            tr.write_line(f"  {r['where']} ({r['dtype']}): max-abs {r['max_abs']:.3e}, "
                          f"lse max-abs {r['lse_max_abs']:.3e} (literal gate)")
    path = os.environ.get("PARITY_LOG_JSON")
    if path:
        import json
        with open(path, "w") as f:
            json.dump(recs, f, indent=1)

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Every attention comparison of the session with its errors (quiet runs included)."""
    from tests.tolerances import BF16_ABS, BF16_REL, F32_REL, RECORDS
    if not RECORDS:
        return
    tr = terminalreporter
    tr.section("attention errors against the float64 oracle")
    tr.write_line(f"bars: f32 row-normwise rel <= {F32_REL:g}; bf16 abs <= {BF16_ABS:g} and "
                  f"row-normwise rel <= {BF16_REL:.4g}")
    for what, dtype, a, r in RECORDS:
        tr.write_line(f"{dtype:5s} abs {a:.3e}  rel {r:.3e}  {what}")

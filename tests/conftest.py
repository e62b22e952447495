import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libmla")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print every GPU parity comparison's error and the margin left under the
    bar, so that a quiet (-q) run still records them."""
    mod = sys.modules.get("gpu_helpers")
    rep = getattr(mod, "REPORT", None) if mod else None
    if not rep:
        return
    tr = terminalreporter
    tr.write_sep("-", "GPU parity: max|err|, max|ref|, margin under the bar, lse max|err|")
    for what, err, ref_max, margin, lerr, n in rep:
        tr.write_line(f"{what}: rows {n} err {err:.3e} ref {ref_max:.3e} margin {margin:.3e} "
                      f"lse {lerr:.3e}")

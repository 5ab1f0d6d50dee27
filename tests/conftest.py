import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the output errors every parity check observed (GPU runs)."""
    try:
        import parity
    except Exception:
        return
    if not parity.STATS:
        return
    tr = terminalreporter
    tr.section("parity: observed errors against the fp64 oracle")
    tr.write_line(f"{'case':58s} {'units':>5s} {'max-abs':>9s} {'mean-abs':>9s} "
                  f"{'max/RMS':>8s} {'/bound':>7s} {'lse':>9s}")
    for st in parity.STATS:
        bound = st.get("bound")
        tr.write_line(f"{st['case'][:58]:58s} {st.get('units', 0):5d} {st.get('max_abs', 0):9.2e} "
                      f"{st.get('mean_abs', 0):9.2e} {st.get('rel', 0):8.4f} "
                      f"{'' if bound is None else format(bound, '7.3f'):>7s} "
                      f"{st.get('lse', 0):9.2e}")

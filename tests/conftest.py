import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """The largest max err / bound of each parity check label, so that the
    observed margins show in the summary of every run (with or without -s)."""
    from tolerance import RATIOS
    if not RATIOS:
        return
    worst = {}
    for label, ratio, count in RATIOS:
        base = label.split(" window")[0]
        r, n = worst.get(base, (0.0, 0))
        worst[base] = (max(r, ratio), n + count)
    terminalreporter.write_sep("-", "parity: max |err| / (tau * m) per check (%d checks)" % len(RATIOS))
    ranked = sorted(worst, key=lambda b: -worst[b][0])
    # the 20 closest to their bound, then every full-size comparison
    shown = ranked[:20] + [b for b in ranked[20:] if "full" in b]
    for base in shown:
        r, n = worst[base]
        terminalreporter.write_line("  %-60s %.3g  (%d elements)" % (base[:60], r, n))

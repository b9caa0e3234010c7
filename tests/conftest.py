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
    config.addinivalue_line("markers", "slow: full-size workloads (seconds to a minute each)")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """List every parity case whose iteration count was accepted through the
    one-off ambiguity band or the float32 count reference, and every
    advancing-window case whose acceptance decisions differed from the float64
    oracle's within the band (none means every count and decision equalled
    the oracle's)."""
    mod = sys.modules.get("_parity")
    if mod is None:
        return
    log = getattr(mod, "BAND_LOG", [])
    terminalreporter.write_line(f"parity counts: {len(log)} case(s) accepted off the float64 oracle's count")
    for label, mode, kind, gw, ow in log:
        terminalreporter.write_line(f"  {label} mode={mode}: {kind}; library {gw[:8]} oracle {ow[:8]}")

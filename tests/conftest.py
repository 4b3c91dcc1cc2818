import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """List the recorded parity statistics (literal max errors, elements admitted only by the
    one-ulp clause) at the end of the run, so that they survive a quiet (-q) run's output."""
    try:
        from parity import BWD_RECORDED, RECORDED
    except ImportError:
        return
    if RECORDED:
        terminalreporter.section("parity against the oracle (rows compared in full)")
        for label, s in RECORDED:
            terminalreporter.write_line(
                f"{label}: n={s['n']} max|dO|={s['max_err_o']:.4e} max|dLSE|={s['max_err_lse']:.3e} "
                f"ulp_clause={s['n_ulp_clause']} fail={s['n_fail_o'] + s['n_fail_lse']} "
                f"rms|dO|/rms|O|={s['rms_err_o'] / max(s['rms_ref_o'], 1e-300):.2e}")
    if BWD_RECORDED:
        terminalreporter.section("backward against the oracle (every element; worst |error| / "
                                 "(|ref| + head rms), then rms error / rms)")
        for label, grads in BWD_RECORDED:
            terminalreporter.write_line(f"{label}: " + " ".join(
                f"{n} {s['max_ratio']:.4f}/{s['rms_ratio']:.4f}" for n, s in grads.items()))

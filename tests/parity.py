"""Comparison of GPU outputs with the CPU oracle (test helper; no attention arithmetic).

The tolerance itself lives in ``oracle/parity.py`` (shared with the bench's parity check): an O
element passes when |O_gpu - O_ref| <= 1.5e-2, or, where |O_ref| >= 2, when it is within one bf16
ulp of O_ref; LSE passes when |LSE_gpu - LSE_ref| <= 1e-3. ``record`` keeps the statistics of
named checks so that the end of a pytest run can print them (``conftest.py``); ``record_bwd`` does
the same for the backward's gradient checks.
"""
from __future__ import annotations

from oracle.parity import LSE_TOL, O_TOL, bf16_ulp, compare, passed  # noqa: F401

# (label, stats) of the checks that asked to be listed in the run's summary
RECORDED: list = []
# (label, {gradient name: stats}) of the backward checks that asked to be listed
BWD_RECORDED: list = []


def record(label: str, stats: dict) -> None:
    RECORDED.append((label, dict(stats)))


def record_bwd(label: str, stats: dict) -> None:
    BWD_RECORDED.append((label, {name: dict(s) for name, s in stats.items()}))


def assert_parity(stats: dict, label: str = ""):
    msg = f"{label}: {stats}"
    assert stats["n_nonfinite"] == 0, msg
    assert stats["n_fail_o"] == 0, msg
    assert stats["n_fail_lse"] == 0, msg

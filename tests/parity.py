"""Comparison of GPU outputs with the CPU oracle (test helper; no attention arithmetic).

The tolerance itself lives in ``oracle/parity.py`` (shared with the bench's parity check): an O
element passes when |O_gpu - O_ref| <= 1.5e-2, or, where |O_ref| >= 2, when it is within one bf16
ulp of O_ref; LSE passes when |LSE_gpu - LSE_ref| <= 1e-3. ``record`` keeps the statistics of
named checks so that the end of a pytest run can print them (``conftest.py``); ``record_bwd`` does
the same for the backward's gradient checks.
"""
from __future__ import annotations

from oracle.parity import LSE_TOL, O_TOL, bf16_ulp, compare, passed  # noqa: F401

# Relative RMS error of O, a check derived from the arithmetic next to the stated element bound
# (which, at |O| ~ 1e-2 as in the non-causal d = 128 workload, would admit errors the size of O). The
# kernel rounds P to bf16 before P.V and O to bf16 at the end. RNE to bf16 (8 significant bits, the
# mantissa fraction uniform) has E[rel^2] = 2^-14 / 24: 2^-7 / sqrt(24) = 1.60e-3 relative RMS from
# the rounding of O. For the workloads' i.i.d. zero-mean V, E[O_c^2] = E[sum_j p_j^2 v_jc^2], so the
# rounding of P adds at most as much (less where a row's top weight, exactly 1, carries the sum), and
# the expected relative RMS error is at most 2^-7 / sqrt(12) = 2.26e-3. The tests allow twice that.
RMS_O_REL = 2.0 * 2.0 ** -7 / 12.0 ** 0.5

# (label, stats) of the checks that asked to be listed in the run's summary
RECORDED: list = []
# (label, {gradient name: stats}) of the backward checks that asked to be listed
BWD_RECORDED: list = []


def record(label: str, stats: dict) -> None:
    RECORDED.append((label, dict(stats)))


def record_bwd(label: str, stats: dict) -> None:
    BWD_RECORDED.append((label, {name: dict(s) for name, s in stats.items()}))


def assert_rms(stats: dict, label: str = ""):
    """The relative RMS check (RMS_O_REL), for outputs of i.i.d. zero-mean V."""
    assert stats["rms_err_o"] <= RMS_O_REL * stats["rms_ref_o"], f"{label}: {stats}"


def assert_parity(stats: dict, label: str = ""):
    msg = f"{label}: {stats}"
    assert stats["n_nonfinite"] == 0, msg
    assert stats["n_fail_o"] == 0, msg
    assert stats["n_fail_lse"] == 0, msg

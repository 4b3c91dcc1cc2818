"""Comparison of GPU outputs with the oracle's — TEST INFRASTRUCTURE ONLY (no attention arithmetic).

Used by ``tests/`` and by the parity check of ``bench.py``'s CPU-baseline leg, which compares the
timed launch's output with the oracle output of the same run.

Tolerance on O (bf16): an element passes when |O_gpu - O_ref| <= 1.5e-2, or, where |O_ref| >= 2,
when it is within one bf16 ulp of O_ref. The second clause exists because at |O| >= 4 the bf16
spacing is 2^-5, so even the correctly rounded exact answer can sit 1.5625e-2 away from it; the
clause admits exactly the two bf16 neighbours of the exact value (and nothing farther). The
literal max error and the number of elements that needed the ulp clause are reported.
Tolerance on LSE (fp32): |LSE_gpu - LSE_ref| <= 1e-3.
``compare`` also reports the RMS of the O error and of O_ref, for the tests' relative RMS check.
"""
from __future__ import annotations

import numpy as np

O_TOL = 1.5e-2
LSE_TOL = 1e-3


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (normal range): 2^(floor(log2|x|) - 7)."""
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def compare(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray) -> dict:
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    err = np.abs(o_gpu - o_ref)
    literal_ok = err <= O_TOL
    ulp_ok = (np.abs(o_ref) >= 2.0) & (err <= bf16_ulp(o_ref))
    ok = literal_ok | ulp_ok
    lerr = np.abs(lse_gpu - lse_ref)
    return {
        "max_err_o": float(err.max()) if err.size else 0.0,
        "max_err_lse": float(lerr.max()) if lerr.size else 0.0,
        "n_ulp_clause": int(np.count_nonzero(ok & ~literal_ok)),
        "n_fail_o": int(np.count_nonzero(~ok)),
        "n_fail_lse": int(np.count_nonzero(~(lerr <= LSE_TOL))),
        "n_nonfinite": int(np.count_nonzero(~np.isfinite(o_gpu)) + np.count_nonzero(~np.isfinite(lse_gpu))),
        "n": int(err.size),
        "rms_err_o": float(np.sqrt(np.mean(err ** 2))) if err.size else 0.0,
        "rms_ref_o": float(np.sqrt(np.mean(np.square(o_ref)))) if err.size else 0.0,
    }


def passed(stats: dict) -> bool:
    return stats["n_nonfinite"] == 0 and stats["n_fail_o"] == 0 and stats["n_fail_lse"] == 0

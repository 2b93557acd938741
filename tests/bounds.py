"""The fp32 rounding-error bound of the parity tests, derived from the
accumulation that forms each output element.

An fp32 evaluation of attention forms every output from sums: dot products of
head_dim terms (scores, dP) and sums over n keys (O, dQ) or n queries (dK, dV).
``oracle.magnitudes`` carries absolute values through the same formulas, so
that each rounding error (at most u = 2^-24 relative) is weighted by the
magnitude of what it rounds: M.  Rounding errors of an n-term sum grow like
sqrt(n) u times the sum of the terms' magnitudes when they behave as
independent random perturbations (the standard probabilistic model), so the
bound on an element is

    |x_gpu - x_ref| <= tol + kappa u M,   kappa = sqrt(n) + sqrt(D),

with n the longer of seq_q and seq_kv (the longest sum) and D the head_dim
(the dot products inside the scores and dP).  tol is the absolute bar (1e-4 on
O, 1e-5 on gradients).  A case passes strictly when its absolute error is
within tol; otherwise it must be within this per-element bound, and the tests
log which of the two held.
"""
from __future__ import annotations

import math

import numpy as np

U32 = 2.0 ** -24


def kappa(seq_q: int, seq_kv: int, head_dim: int) -> float:
    return math.sqrt(max(seq_q, seq_kv)) + math.sqrt(head_dim)


def within(err: np.ndarray, tol: float, kap: float, mag: np.ndarray):
    """(ok, worst ratio of err to the per-element bound)."""
    bound = tol + kap * U32 * mag
    if not err.size:
        return True, 0.0
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    ratio = float(r.max())
    return ratio <= 1.0, ratio

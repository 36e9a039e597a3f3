"""Oracle of the latency-model fit (TEST INFRASTRUCTURE ONLY; used by the
test-suite and by nothing in the library).

BASTION, "Methodik" §3, latency modelling: the verification latency
T_verify(N) of a tree of N draft nodes follows a roofline-shaped model
(memory bandwidth, then compute) calibrated on observed runtimes; the pages'
controller divides by C(N).  Reading: C(N) = a + b N + c max(0, N - knee),
the knee where verification turns compute-bound, fitted to measured
(N, time) pairs by least squares: for every integer knee in the given range
the three coefficients come from a library least-squares solve, and the knee
with the smallest residual sum of squares wins (equal sums: the smaller
knee).  A knee at or beyond every measured N leaves c undetermined; it is
fitted with c = 0.
"""
from __future__ import annotations

import numpy as np


def fit_cost(n, t, knee_min, knee_max):
    """Returns (a, b, c, knee, rss)."""
    n = np.asarray(n, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    best = None
    for knee in range(int(knee_min), int(knee_max) + 1):
        hinge = np.maximum(0.0, n - knee)
        if np.any(hinge > 0):
            X = np.stack([np.ones_like(n), n, hinge], axis=1)
            coef, *_ = np.linalg.lstsq(X, t, rcond=None)
            a, b, c = coef
        else:
            X = np.stack([np.ones_like(n), n], axis=1)
            (a, b), *_ = np.linalg.lstsq(X, t, rcond=None)
            c = 0.0
        rss = float(np.sum((a + b * n + c * hinge - t) ** 2))
        if best is None or rss < best[4] * (1 - 1e-12) - 1e-300:
            best = (float(a), float(b), float(c), knee, rss)
    return best

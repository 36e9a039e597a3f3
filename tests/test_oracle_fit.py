"""Pins of the latency-model fit oracle (oracle/fit.py): noiseless
piecewise-linear data is recovered exactly (closed form), a straight line
gives c = 0 at any knee the data cannot see, and symmetric noise does not
move the knee."""
import numpy as np
import pytest

from oracle.fit import fit_cost

NS = np.array([0, 1, 2, 4, 8, 12, 16, 24, 32, 40, 48, 56, 64, 80, 96, 112, 128], float)


@pytest.mark.parametrize("a,b,c,knee", [(10.0, 0.05, 0.3, 32), (150.0, 0.01, 2.0, 80),
                                        (3.0, 0.2, 0.0, 40), (1.0, 0.005, 0.03, 32)])
def test_recovers_piecewise_linear(a, b, c, knee):
    t = a + b * NS + c * np.maximum(0, NS - knee)
    fa, fb, fc, fk, rss = fit_cost(NS, t, 0, 128)
    assert rss < 1e-18 * max(1.0, a * a)
    assert fa == pytest.approx(a, rel=1e-9)
    assert fb == pytest.approx(b, rel=1e-7, abs=1e-12)
    assert fc == pytest.approx(c, rel=1e-7, abs=1e-12)
    if c > 0:
        assert fk == knee


def test_straight_line_has_no_hinge():
    t = 5.0 + 0.1 * NS
    fa, fb, fc, fk, rss = fit_cost(NS, t, 0, 128)
    assert abs(fc) < 1e-9 and fb == pytest.approx(0.1, rel=1e-9)


def test_knee_under_symmetric_noise():
    rng = np.random.default_rng(0)
    t = 20.0 + 0.02 * NS + 0.5 * np.maximum(0, NS - 48)
    noisy = np.repeat(t, 2) + np.tile([1e-3, -1e-3], len(t))
    fa, fb, fc, fk, rss = fit_cost(np.repeat(NS, 2), noisy, 0, 128)
    assert fk == 48 and fc == pytest.approx(0.5, rel=1e-6)

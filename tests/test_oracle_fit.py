"""Pins of the verify cost fit (thinkspread, 'The economics of speculative
decoding': time(m) = fixed + marginal * m)."""
import numpy as np
import pytest

from oracle.fit import fit_fixed_marginal


def test_exact_line_is_recovered():
    a, b, r2 = fit_fixed_marginal(range(1, 9), [9.0 + 5.5 * m for m in range(1, 9)])
    assert a == pytest.approx(9.0, abs=1e-12)
    assert b == pytest.approx(5.5, abs=1e-12)
    assert r2 == pytest.approx(1.0, abs=1e-12)


def test_matches_numpy_polyfit():
    g = np.random.default_rng(3)
    m = np.arange(1, 9)
    t = 3.0 + 0.2 * m + g.normal(0, 0.05, 8)
    a, b, _ = fit_fixed_marginal(m, t)
    pb, pa = np.polyfit(m, t, 1)
    assert a == pytest.approx(pa, abs=1e-12) and b == pytest.approx(pb, abs=1e-12)


def test_flat_cost_has_zero_marginal():
    a, b, r2 = fit_fixed_marginal([1, 2, 3], [4.0, 4.0, 4.0])
    assert (a, b, r2) == (4.0, 0.0, 1.0)

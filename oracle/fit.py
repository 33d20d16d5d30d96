"""Oracle: the fixed + marginal-per-row cost model of verification.

Test infrastructure only (see ``oracle/__init__.py``).

thinkspread, "The economics of speculative decoding", opening section: verify
time is modelled as a fixed term plus a per-row term, time(m) = a + b*m with
m = k + 1 rows. Here a and b come from ordinary least squares.
"""
from __future__ import annotations

import numpy as np


def fit_fixed_marginal(m_values, times):
    """Least-squares (a, b, r2) of times ~ a + b*m."""
    m = np.asarray(m_values, dtype=np.float64)
    t = np.asarray(times, dtype=np.float64)
    mb, tb = m.mean(), t.mean()
    sxx = ((m - mb) ** 2).sum()
    b = ((m - mb) * (t - tb)).sum() / sxx
    a = tb - b * mb
    ss_res = ((t - (a + b * m)) ** 2).sum()
    ss_tot = ((t - tb) ** 2).sum()
    r2 = 1.0 - ss_res / ss_tot if ss_tot > 0 else 1.0
    return float(a), float(b), float(r2)

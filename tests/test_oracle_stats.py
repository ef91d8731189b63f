"""Pins of the oracle's per-stage statistics (the traced forward's summary of one stage's values; CPU only).

Hand-worked vectors with NaN and infinities, the all-non-finite and empty cases, and agreement with numpy's own
reductions on a large random vector (min, max, mean and root mean square over the finite values; NaN and Inf
counts), so a statistic taken over the wrong set or a swapped field fails.
"""
import math

import numpy as np

import oracle


def test_hand_worked_vector():
    s = oracle.stage_stats([1.0, 2.0, float("nan"), -math.inf, 3.0, math.inf])
    n, nan, inf, mn, mx, mean, rms = s
    assert (n, nan, inf) == (6, 1, 2)
    assert (mn, mx) == (1.0, 3.0)
    assert mean == 2.0
    assert abs(rms - math.sqrt(14.0 / 3.0)) < 1e-15


def test_negative_values_and_single_value():
    s = oracle.stage_stats([-4.0])
    assert list(s) == [1, 0, 0, -4.0, -4.0, -4.0, 4.0]
    s = oracle.stage_stats([-1.0, -5.0, 2.0])
    assert (s[3], s[4]) == (-5.0, 2.0)
    assert abs(s[5] - (-4.0 / 3.0)) < 1e-15
    assert abs(s[6] - math.sqrt(30.0 / 3.0)) < 1e-15


def test_no_finite_values():
    s = oracle.stage_stats([float("nan"), math.inf])
    assert list(s) == [2, 1, 1, 0.0, 0.0, 0.0, 0.0]
    assert list(oracle.stage_stats([])) == [0, 0, 0, 0.0, 0.0, 0.0, 0.0]


def test_agrees_with_numpy_reductions():
    g = np.random.default_rng(3)
    v = g.standard_normal(100_000) * 7.0 + 1.5
    v[g.choice(v.size, 13, replace=False)] = np.nan
    v[g.choice(v.size, 5, replace=False)] = np.inf
    s = oracle.stage_stats(v)
    fin = v[np.isfinite(v)]
    assert s[0] == v.size and s[1] == np.isnan(v).sum() and s[2] == np.isinf(v).sum()
    assert s[3] == fin.min() and s[4] == fin.max()
    assert abs(s[5] - fin.mean()) < 1e-12 * np.abs(fin).max()
    assert abs(s[6] - np.sqrt(np.mean(fin * fin))) < 1e-12 * s[6]

"""Pins for the Sequential Temperature Scaling fit.

Pages: summary page §3.2.1 (STS calibrates the cumulative prefix survival on
held-out data; a left-to-right one-dimensional grid search chooses each
position's temperature to minimise that position's Expected Calibration
Error with the earlier positions' calibration held fixed) and §4.3.3 (the
reported ECE falls after STS).

Pins: the ECE of hand-built bins computed with exact fractions; a perfectly
calibrated model recovers T = 1 at every position; data drawn with known,
different per-position temperatures recovers them (a fit that ignored the
earlier positions' calibration, planted below, does not); the first
position's choice ignores later positions; rollout order does not matter;
the fitted ECE never exceeds the ECE at T = 1.
"""
from fractions import Fraction

import numpy as np
import pytest


def _exact_ece_units(a, y, M):
    """N * ECE in units of 2^-40 from the definition, with exact fractions."""
    acc = [Fraction(0)] * M
    for ai, yi in zip(a, y):
        b = min(int(Fraction(float(ai)) * M), M - 1)
        units = round(Fraction(float(ai)) * 2 ** 40)  # ties cannot occur for these values
        acc[b] += (int(yi) << 40) - units
    return int(sum(abs(x) for x in acc))


def test_ece_hand_bins(oracle):
    a = np.array([0.1, 0.1, 0.9, 0.9, 0.5, 0.5, 0.25], np.float32)
    y = np.array([0, 1, 1, 1, 1, 0, 0], np.uint8)
    for M in (1, 4, 10, 15):
        assert oracle.ece_units(a, y, M) == _exact_ece_units(a, y, M)
    # calibrated bins: two values of 0.5 with one success each -> 0 in that bin
    assert oracle.ece_units(np.array([0.5, 0.5], np.float32), np.array([1, 0], np.uint8), 10) == 0
    # one bin: |sum(y) - sum(a)|
    assert oracle.ece_units(a, y, 1) == abs((int(y.sum()) << 40) - sum(round(float(x) * 2 ** 40) for x in a))


def _rollouts(rng, N, t_true, mu=1.5, sd=1.5):
    """Scores and survival labels of a model whose true acceptance at position
    j is sigmoid(s / t_true[j]), each position conditional on the earlier ones
    (labels: all positions up to j accepted)."""
    gamma = len(t_true)
    s = rng.normal(mu, sd, (N, gamma))
    c = 1.0 / (1.0 + np.exp(-s / np.asarray(t_true)[None, :]))
    acc = rng.random((N, gamma)) < c
    return s, np.cumprod(acc, axis=1).astype(np.uint8)


GRID = np.round(np.arange(0.40, 3.01, 0.05), 10)


def test_calibrated_model_keeps_unit_temperature(oracle):
    rng = np.random.default_rng(21)
    s, y = _rollouts(rng, 200_000, [1.0] * 5)
    r = oracle.sts_fit(s, y, GRID, bins=15)
    assert np.all(np.abs(r["temps"] - 1.0) <= 0.101), r["temps"]


def test_recovers_per_position_temperatures(oracle):
    rng = np.random.default_rng(22)
    t_true = [0.7, 1.4, 2.0, 1.0]
    s, y = _rollouts(rng, 200_000, t_true)
    r = oracle.sts_fit(s, y, GRID, bins=15)
    assert np.all(np.abs(r["temps"] - np.array(t_true)) <= 0.151), r["temps"]
    assert np.all(r["ece_units"] <= r["ece1_units"])
    # the calibrated survival is the product of the calibrated confidences
    # (numpy's exp may differ from the C library's in the last bit)
    T = np.array([GRID[np.argmin(np.abs(GRID - t))] for t in r["temps"]])
    c = (1.0 / (1.0 + np.exp(-s / T[None, :]))).astype(np.float32)
    np.testing.assert_allclose(r["a"], np.cumprod(c, axis=1, dtype=np.float32), rtol=1e-6, atol=0)


def test_planted_non_sequential_fit_fails(oracle):
    """Fitting each position against T = 1 survival of the earlier positions
    (not holding their calibrated values) misses the true temperatures: the
    recovery pin above would catch that mistake."""
    rng = np.random.default_rng(23)
    t_true = [0.7, 1.4, 2.0, 1.0]
    s, y = _rollouts(rng, 200_000, t_true)
    N, gamma = s.shape
    wrong = []
    prev = np.ones(N, np.float32)
    for j in range(gamma):
        best = None
        for T in GRID:
            c = (1.0 / (1.0 + np.exp(-s[:, j] / T))).astype(np.float32)
            e = oracle.ece_units(prev * c, y[:, j], 15)
            if best is None or e < best[0]:
                best = (e, T)
        wrong.append(best[1])
        prev = prev * (1.0 / (1.0 + np.exp(-s[:, j]))).astype(np.float32)  # the planted mistake
    assert np.any(np.abs(np.array(wrong) - np.array(t_true)) > 0.151), wrong


def test_first_position_ignores_later_ones(oracle):
    rng = np.random.default_rng(24)
    s, y = _rollouts(rng, 20_000, [1.2, 0.8, 1.6])
    r1 = oracle.sts_fit(s, y, GRID)
    s2 = s.copy()
    s2[:, 1:] = rng.normal(0.0, 3.0, s2[:, 1:].shape)
    y2 = y.copy()
    y2[:, 1:] = y2[:, :1] * (rng.random(y2[:, 1:].shape) < 0.5)
    r2 = oracle.sts_fit(s2, y2, GRID)
    assert r1["temps"][0] == r2["temps"][0] and r1["ece_units"][0] == r2["ece_units"][0]


def test_rollout_order_does_not_matter(oracle):
    rng = np.random.default_rng(25)
    s, y = _rollouts(rng, 5_000, [1.3, 0.9])
    r1 = oracle.sts_fit(s, y, GRID)
    p = rng.permutation(s.shape[0])
    r2 = oracle.sts_fit(s[p], y[p], GRID)
    np.testing.assert_array_equal(r1["temps"], r2["temps"])
    np.testing.assert_array_equal(r1["ece_units"], r2["ece_units"])
    np.testing.assert_array_equal(r1["a"][p], r2["a"])


def test_grid_of_copies_of_one(oracle):
    """A grid holding only T = 1 (repeated: exact ties) fits T = 1 with the ECE
    at T = 1."""
    rng = np.random.default_rng(26)
    s, y = _rollouts(rng, 5_000, [1.0])
    r = oracle.sts_fit(s, y, np.array([1.0, 1.0, 1.0]))
    assert r["temps"][0] == 1.0 and r["ece_units"][0] == r["ece1_units"][0]

"""Pins for prefix-survival products and Algorithm 1 (hardware-aware prefix scheduler).

Pages: summary page §3.2.2 (a_{r,j} = prod c_{r,i}; B = sum(1 + l_r);
tau = sum(1 + sum_{j<=l_r} a_{r,j}); Theta = tau * SPS(B); candidates taken in
order of survival probability, which respects prefixes and maximises expected
accepted tokens at fixed B; causal stop at the first non-improvement, which
finds the global maximum when Theta is unimodal along the path) and 5.2.
Pins: numpy's binary32 cumulative product, brute force over every length
vector for tiny R and gamma, the unimodal-path global optimum, and
non-anticipation under perturbation of later positions.
"""
import itertools

import numpy as np
import pytest


def test_prefix_products_match_numpy_cumprod(oracle):
    rng = np.random.default_rng(0)
    c = rng.random((50, 16)).astype(np.float32)
    c[3, 4] = 1.0
    c[7, 0] = 0.0
    a = oracle.prefix_products(c)
    np.testing.assert_array_equal(a, np.cumprod(c, axis=1, dtype=np.float32))
    assert np.all(np.diff(a, axis=1) <= 0) and np.all((a >= 0) & (a <= 1))


def _all_lengths(R, gamma):
    return itertools.product(range(gamma + 1), repeat=R)


def _tau(a, L):
    return sum(1.0 + float(np.sum(a[r, :L[r]], dtype=np.float64)) for r in range(len(L)))


def _rand_case(rng, R, gamma, n_sps):
    c = rng.uniform(0.05, 1.0, (R, gamma)).astype(np.float32)
    a = np.cumprod(c, axis=1, dtype=np.float32)
    return a


def test_greedy_order_maximises_tau_at_fixed_B(oracle):
    """Every point of the survival-ordered path reaches the largest tau among all
    prefix-respecting length vectors with the same batch size B."""
    rng = np.random.default_rng(1)
    for trial in range(40):
        R, gamma = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        a = _rand_case(rng, R, gamma, R * (gamma + 1))
        best = {}
        for L in _all_lengths(R, gamma):
            B = R + sum(L)
            best[B] = max(best.get(B, -1.0), _tau(a, L))
        # SPS constant: Theta = tau * 1 strictly grows along the whole path
        s = oracle.schedule(a, np.ones(R * (gamma + 1), np.float32))
        path = s["theta_path"]
        assert s["n_sel"] == R * gamma
        for i in range(R * gamma + 1):
            assert path[i] == pytest.approx(best[R + i], rel=1e-9)


def _theta_all(a, sps, R, gamma):
    out = {}
    for L in _all_lengths(R, gamma):
        B = R + sum(L)
        out[L] = _tau(a, L) * float(sps[B - 1])
    return out


def test_unimodal_path_reaches_global_maximum(oracle):
    rng = np.random.default_rng(2)
    checked = 0
    for trial in range(300):
        R, gamma = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        if (gamma + 1) ** R > 4000:
            continue
        a = _rand_case(rng, R, gamma, R * (gamma + 1))
        B = np.arange(1, R * (gamma + 1) + 1)
        knee = rng.integers(1, R * (gamma + 1) + 1)
        sps = (1000.0 * np.minimum(1.0, knee / B) * rng.uniform(0.9, 1.0)).astype(np.float32)
        s = oracle.schedule(a, sps)
        # the full survival-ordered path, built with a library sort
        order = np.lexsort((np.tile(np.arange(1, gamma + 1), R), np.repeat(np.arange(R), gamma), -a.ravel()))
        taus = R + np.concatenate([[0.0], np.cumsum(a.ravel()[order].astype(np.float64))])
        path = np.array([taus[i] * float(sps[R + i - 1]) for i in range(R * gamma + 1)])
        peak = int(np.argmax(path))
        unimodal = np.all(np.diff(path[:peak + 1]) > 0) and np.all(np.diff(path[peak:]) <= 0)
        glob = max(_theta_all(a, sps, R, gamma).values())
        if unimodal:
            checked += 1
            assert s["stats"][2] == pytest.approx(glob, rel=1e-9)
        assert s["stats"][2] <= glob * (1 + 1e-9)
    assert checked > 50


def test_stop_is_causal_and_respects_prefixes(oracle):
    """[l_r >= j] does not change when c_{r,j+1..gamma} change (non-anticipation),
    and B, tau and Theta agree with the selected lengths."""
    rng = np.random.default_rng(3)
    for trial in range(60):
        R, gamma = int(rng.integers(2, 7)), int(rng.integers(2, 7))
        c = rng.uniform(0.2, 1.0, (R, gamma)).astype(np.float32)
        B = np.arange(1, R * (gamma + 1) + 1)
        sps = (1000.0 * np.minimum(1.0, (R + rng.integers(0, R * gamma + 1)) / B)).astype(np.float32)
        s = oracle.schedule(oracle.prefix_products(c), sps)
        L = s["lengths"]
        a = oracle.prefix_products(c)
        assert s["stats"][0] == R + L.sum()
        assert s["stats"][1] == pytest.approx(_tau(a, L), rel=1e-10)
        assert s["stats"][2] == pytest.approx(_tau(a, L) * float(sps[R + L.sum() - 1]), rel=1e-10)
        for r in range(R):
            for j in range(1, gamma + 1):
                c2 = c.copy()
                c2[r, j:] = rng.uniform(0.0, 1.0, gamma - j).astype(np.float32)
                L2 = oracle.schedule(oracle.prefix_products(c2), sps)["lengths"]
                assert (L2[r] >= j) == (L[r] >= j)


def test_theta_path_and_stop_gap(oracle):
    a = np.array([[0.9, 0.5], [0.8, 0.1]], np.float32)
    sps = np.array([1, 1, 1, 0.6, 0.5, 0.4], np.float32) * 100
    s = oracle.schedule(a, sps)
    # path: theta0 = 2*100; +0.9 (B=3) -> 290; +0.8 (B=4) -> 3.7*60 = 222 <= 290: stop
    assert s["theta_path"][0] == pytest.approx(200.0)
    assert s["theta_path"][1] == pytest.approx(290.0, rel=1e-7)
    assert s["theta_path"][2] == pytest.approx(222.0, rel=1e-6)
    assert np.isnan(s["theta_path"][3])
    assert list(s["lengths"]) == [1, 0]
    assert s["stop_gap"] == pytest.approx((290 - 222) / 290, rel=1e-6)


def test_tau_units_round_to_nearest(oracle):
    assert oracle.tau_units(1.0) == 2 ** 38
    assert oracle.tau_units(0.5) == 2 ** 37
    assert oracle.tau_units(0.0) == 0
    assert oracle.tau_units(2.0 ** -40) == 0           # quarter unit rounds down
    assert oracle.tau_units(3 * 2.0 ** -39) == 2       # 1.5 units: ties to even


def test_short_sps_table_is_rejected(oracle):
    with pytest.raises(ValueError):
        oracle.schedule(np.ones((2, 3), np.float32), np.ones(7, np.float32))

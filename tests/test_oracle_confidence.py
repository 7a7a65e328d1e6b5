"""Pins for the oracle's confidence head with per-position temperatures (STS).

Pages: summary page §3.2.1 (c_k predicted from the backbone state h_k and the
Markov embedding of x_{k-1}; STS rescales per position).  The readings
(logit = w . [h_k; W1[x_{k-1}]], no bias; c = sigmoid(logit / T_k)) are
pinned to scipy's expit and numpy's dot product, with T_k = 1 as identity.
"""
import numpy as np
from scipy import special


def test_confidence_matches_expit_of_dot(oracle):
    rng = np.random.default_rng(0)
    R, gamma, H, V, rank = 3, 4, 64, 50, 16
    h = rng.standard_normal((R, gamma, H)).astype(np.float32)
    W1 = rng.standard_normal((V, rank)).astype(np.float32)
    w = rng.standard_normal(H + rank).astype(np.float32) * 0.1
    temps = np.array([0.8, 1.0, 1.2, 1.5], np.float32)
    anchors = rng.integers(0, V, R).astype(np.int32)
    tokens = rng.integers(0, V, (R, gamma)).astype(np.int32)
    c = oracle.confidence(h, w, temps, W1, anchors, tokens)
    for r in range(R):
        for k in range(gamma):
            prev = anchors[r] if k == 0 else tokens[r, k - 1]
            s = np.dot(w.astype(np.float64), np.concatenate([h[r, k], W1[prev]]).astype(np.float64))
            assert c[r, k] == np.float32(special.expit(s / float(temps[k])))


def test_unit_temperature_and_monotonicity(oracle):
    rng = np.random.default_rng(1)
    H, V, rank = 8, 10, 4
    W1 = np.zeros((V, rank), np.float32)
    w = np.ones(H + rank, np.float32)
    h = np.linspace(-3, 3, 7, dtype=np.float32)[:, None, None] * np.ones((1, 1, H), np.float32)
    c = oracle.confidence(h, w, np.ones(1, np.float32), W1, np.zeros(7, np.int32), np.zeros((7, 1), np.int32))
    np.testing.assert_allclose(c[:, 0], special.expit(H * np.linspace(-3, 3, 7)), rtol=1e-6)
    assert np.all(np.diff(c[:, 0]) > 0)

"""Pins for the oracle's verification stage (standard speculative rejection
sampling with resample and bonus token, plus the analytic acceptance c*).

Pages: summary page 요약 and §3.2.1 (c*_k = 1 - 1/2 ||p^d_k - p^t_k||_1);
notes page 배경 (the target keeps the longest accepted prefix by rejection
sampling, preserving its distribution).  Pins: closed forms of c*, exact
enumeration over the draft token and a fine uniform grid showing that the
output marginal equals p^t and that P(accept) = c*, a statistical check of the
emitted chain against a prefix-dependent target, and the Appendix A example.
"""
import json
import os

import numpy as np
import pytest
from scipy import special, stats

HERE = os.path.dirname(os.path.abspath(__file__))


def _logp(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, np.float64))


def test_cstar_closed_forms(oracle):
    p = np.array([0.2, 0.3, 0.5])
    assert oracle.cstar(_logp(p), _logp(p)) == pytest.approx(1.0, abs=1e-15)
    assert oracle.cstar(_logp([0.5, 0.5, 0, 0]), _logp([0, 0, 0.4, 0.6])) == 0.0
    # the summary page's Appendix A pair: draft (0.5, 0.5) vs target (0.7, 0.3) -> 0.8 = a_1
    assert oracle.cstar(_logp([0.5, 0.5]), _logp([0.7, 0.3])) == pytest.approx(0.8, abs=1e-15)
    rng = np.random.default_rng(0)
    for _ in range(50):
        pd = rng.dirichlet(np.ones(20))
        pt = rng.dirichlet(np.ones(20))
        assert oracle.cstar(_logp(pd), _logp(pt)) == pytest.approx(1 - 0.5 * np.abs(pd - pt).sum(), abs=1e-13)


def _enumerate_block_output(oracle, pd, pt, pt_next, grid=20_000):
    """Exact law of the first emitted token for a one-position verify (length 1),
    enumerating the draft token x ~ p^d and a midpoint grid of the uniform u.
    Returns (P(output = y), P(accept))."""
    V = pd.size
    lpd, lpt = _logp(pd), _logp(pt)
    u = (np.arange(grid) + 0.5) / grid
    lnu = np.log(u)
    logw, npos = oracle.residual_logw(lpd, lpt)
    resid = special.softmax(logw) if npos else pt
    out = np.zeros(V)
    acc_total = 0.0
    for x in range(V):
        if pd[x] == 0:
            continue
        acc = np.mean([oracle.accept(float(l), float(lpt[x]), float(lpd[x])) for l in lnu])
        acc_total += pd[x] * acc
        out[x] += pd[x] * acc
        out += pd[x] * (1 - acc) * resid
    return out, acc_total


def test_output_marginal_equals_target_by_enumeration(oracle):
    rng = np.random.default_rng(1)
    for V in [2, 3, 5]:
        for _ in range(3):
            pd = rng.dirichlet(np.ones(V))
            pt = rng.dirichlet(np.ones(V))
            out, acc = _enumerate_block_output(oracle, pd, pt, None)
            np.testing.assert_allclose(out, pt, atol=2e-4)
            assert acc == pytest.approx(oracle.cstar(_logp(pd), _logp(pt)), abs=2e-4)


def test_enumeration_detects_a_wrong_residual(oracle):
    """Control for the enumeration pin: residual max(0, p^d - p^t) breaks it."""
    pd, pt = np.array([0.6, 0.3, 0.1]), np.array([0.2, 0.3, 0.5])
    lpd, lpt = _logp(pd), _logp(pt)
    wrong = special.softmax(oracle.residual_logw(lpt, lpd)[0])
    right = special.softmax(oracle.residual_logw(lpd, lpt)[0])
    out = {}
    for name, resid in [("wrong", wrong), ("right", right)]:
        o = np.zeros(3)
        for x in range(3):
            a = min(1.0, pt[x] / pd[x])
            o[x] += pd[x] * a
            o += pd[x] * (1 - a) * resid
        out[name] = o
    np.testing.assert_allclose(out["right"], pt, atol=1e-12)
    assert np.abs(out["wrong"] - pt).max() > 0.1


def _run_chain(oracle, R, V, gamma, seed, target_table, draft_logits, lengths=None):
    """Draft with fixed per-position logits (no head bias), then build the target
    rows from the drafted prefix (T_k depends on x_{k-1}) and verify."""
    U = np.tile(draft_logits.astype(np.float32), (R, 1, 1))        # [R, gamma, V]
    W1 = np.zeros((V, 4), np.float32)
    W2 = np.zeros((4, V), np.float32)
    anchors = np.zeros(R, np.int32)
    d = oracle.draft(U, W1, W2, anchors, seed=seed)
    tokens = d["tokens"]
    T = np.zeros((R, gamma + 1, V), np.float32)
    prev = anchors
    for k in range(gamma + 1):
        T[:, k, :] = target_table[k][prev]
        if k < gamma:
            prev = tokens[:, k]
    v = oracle.verify(U, W1, W2, anchors, tokens, T, lengths, seed=seed, chunk=4096)
    return d, v


def test_emitted_chain_follows_prefix_dependent_target(oracle):
    """The emitted tokens follow the target chain: the first emitted token has
    law p^t_1, and given an accepted first token a, the second has law p^t_2(.|a)."""
    V, gamma, R = 3, 2, 60_000
    rng = np.random.default_rng(2)
    draft_logits = rng.standard_normal((gamma, V))
    # target_table[k][prev] = logits of p^t_{k+1}(. | x_k = prev); anchor = 0
    table = [rng.standard_normal((V, V)) * 1.5 for _ in range(gamma + 1)]
    d, v = _run_chain(oracle, R, V, gamma, 21, table, draft_logits)
    n = v["n_accept"]
    first = np.where(n >= 1, d["tokens"][:, 0], v["out_token"])
    p1 = special.softmax(table[0][0])
    assert stats.chisquare(np.bincount(first, minlength=V), R * p1).pvalue > 1e-4
    for a in range(V):
        sel = (n >= 1) & (d["tokens"][:, 0] == a)
        second = np.where(n[sel] >= 2, d["tokens"][sel, 1], v["out_token"][sel])
        p2 = special.softmax(table[1][a])
        assert stats.chisquare(np.bincount(second, minlength=V), sel.sum() * p2).pvalue > 1e-4
    # acceptance rate at position 1 equals c*_1
    pd1 = special.softmax(draft_logits[0])
    c1 = 1 - 0.5 * np.abs(pd1 - p1).sum()
    acc1 = (n >= 1).mean()
    assert abs(acc1 - c1) < 5 * np.sqrt(c1 * (1 - c1) / R)
    np.testing.assert_allclose(v["cstar"][:, 0], c1, atol=1e-6)


def test_zero_length_draws_bonus_from_first_target_row(oracle):
    V, gamma, R = 4, 3, 40_000
    rng = np.random.default_rng(3)
    draft_logits = rng.standard_normal((gamma, V))
    table = [rng.standard_normal((V, V)) for _ in range(gamma + 1)]
    d, v = _run_chain(oracle, R, V, gamma, 5, table, draft_logits, lengths=np.zeros(R, np.int32))
    assert np.all(v["n_accept"] == 0)
    assert np.all(np.isnan(v["cstar"]))
    assert np.all(v["accept_mask"] == 255)
    p1 = special.softmax(table[0][0])
    assert stats.chisquare(np.bincount(v["out_token"], minlength=V), R * p1).pvalue > 1e-4


def test_full_acceptance_draws_bonus_from_next_row(oracle):
    """When the draft equals the target every token is accepted and the bonus
    comes from the row after the verified length."""
    V, gamma, R = 5, 3, 20_000
    rng = np.random.default_rng(4)
    draft_logits = rng.standard_normal((gamma, V))
    bonus = rng.standard_normal(V)
    table = [np.tile(draft_logits[k], (V, 1)) for k in range(gamma)] + [np.tile(bonus, (V, 1))]
    for L in [1, 3]:
        d, v = _run_chain(oracle, R, V, gamma, 8, table, draft_logits, lengths=np.full(R, L, np.int32))
        assert np.all(v["n_accept"] == L)
        np.testing.assert_allclose(v["cstar"][:, :L], 1.0, atol=1e-6)
        nxt = special.softmax(table[L][0])
        assert stats.chisquare(np.bincount(v["out_token"], minlength=V), R * nxt).pvalue > 1e-4


def test_appendix_a_retroactive_counterexample(oracle):
    """Summary page, 부록: a retroactive scheduler biases the output to (0.85, 0.15);
    the causal Algorithm 1 stops at length 0 and the output is the target (0.7, 0.3)."""
    g = json.load(open(os.path.join(HERE, "golden", "appendix_a.json")))
    sps = np.array(g["sps"], np.float32)
    pd, pt = np.array(g["draft_first_position"]), np.array(g["target_first_position"])
    assert oracle.cstar(_logp(pd), _logp(pt)) == pytest.approx(g["a1"], abs=1e-15)

    def theta(lengths, a):
        B = 1 + lengths
        tau = 1 + a[:lengths].sum()
        return tau * float(sps[B - 1])

    def retroactive(c2):           # global max over all lengths after seeing c2
        a = np.array([g["a1"], g["a1"] * c2])
        return int(np.argmax([theta(L, a) for L in range(3)]))

    assert retroactive(g["c2_if_first_token_is_A"]) == g["retroactive_length_for_c2"]["0.9"]
    assert retroactive(g["c2_if_first_token_is_B"]) == g["retroactive_length_for_c2"]["0.0"]
    # causal Algorithm 1 (oracle): theta0 = 1.0, theta1 = 0.9 -> stop at length 0, whatever c2 is
    for c2 in [g["c2_if_first_token_is_A"], g["c2_if_first_token_is_B"]]:
        a = oracle.prefix_products(np.array([[g["a1"], c2]], np.float32))
        s = oracle.schedule(a, sps)
        assert s["lengths"][0] == 0
        assert s["theta_path"][0] == pytest.approx(g["theta0"], rel=1e-7)
        assert s["theta_path"][1] == pytest.approx(g["theta1"], rel=1e-7)
        # derived: theta2 = (1 + 0.8 + 0.8 c2) * 0.45
        assert theta(2, np.array([0.8, 0.8 * c2])) == pytest.approx((1.8 + 0.8 * c2) * 0.45, rel=1e-7)

    # output law of the first emitted token, by enumeration of x1 and the uniform grid
    lpd, lpt = _logp(pd), _logp(pt)
    grid = (np.arange(20_000) + 0.5) / 20_000
    resid = special.softmax(oracle.residual_logw(lpd, lpt)[0])

    def emitted(length, x1):
        if length == 0:            # bonus from p^t_1
            return pt.copy()
        acc = np.mean([oracle.accept(float(np.log(u)), float(lpt[x1]), float(lpd[x1])) for u in grid])
        out = (1 - acc) * resid
        out[x1] += acc
        return out

    c2_of = {0: g["c2_if_first_token_is_A"], 1: g["c2_if_first_token_is_B"]}
    retro = sum(pd[x] * emitted(retroactive(c2_of[x]), x) for x in range(2))
    causal = sum(pd[x] * emitted(0, x) for x in range(2))
    np.testing.assert_allclose(retro, g["retroactive_output"], atol=1e-4)
    np.testing.assert_allclose(causal, pt, atol=1e-12)

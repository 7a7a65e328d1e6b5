"""Shared helpers for the GPU-vs-oracle parity tests.

Inputs come only from the seeded generators (draft_sampling_verification_w1_amd.synth);
target logits that depend on drafted tokens are built from the ORACLE's draft
logits, so no oracle input is derived from the HIP path.  Comparisons follow
the stated bar: token ids, accepted lengths, schedules and bonus tokens bit
exact except where the oracle's own margin is below 1e-6 (a near-tie, logged
and counted); floating-point outputs within rtol 1e-4 / atol 1e-6.
"""
from __future__ import annotations

import sys

import numpy as np

from draft_sampling_verification_w1_amd import synth
from oracle import oracle as O

RTOL, ATOL, TIE = 1e-4, 1e-6, 1e-6

# Running totals over every GPU comparison of the session: draws compared
# (draft tokens, acceptance decisions, final draws), near-ties among them, and
# the largest deviations of the normalisers and of the acceptance log-ratio
# from the oracle's.  The last GPU test of the session checks the tie budget.
STATS = {"draws": 0, "ties": 0, "max_lse_d_err": 0.0, "max_lse_t_err": 0.0,
         "max_rho_err": 0.0, "max_logpd_err": 0.0, "logpd_values": 0}


def _track(key, value):
    if np.isfinite(value) and value > STATS[key]:
        STATS[key] = float(value)


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gen_inputs(cfg: synth.Config):
    W1, W2 = synth.weights(cfg)
    U, Ub = synth.backbone(cfg)
    return {"W1": W1, "W2": W2, "anchors": synth.anchors(cfg), "U": U, "Ub": Ub}


def build_target(cfg, inp, tokens, requests_from_oracle=None):
    """T [R, gamma+1, V] in storage type.  Rows of requests in
    ``requests_from_oracle`` (default: all) use the oracle's draft logits as
    base where the config builds its target from them; other requests use the
    backbone rows U (a draft-independent stand-in, never compared)."""
    R, g, V = cfg.R, cfg.gamma, cfg.V
    dt = np.uint16 if cfg.dtype == "bf16" else np.float32
    T = np.empty((R, g + 1, V), dt)
    req = set(range(R)) if requests_from_oracle is None else set(int(r) for r in requests_from_oracle)
    W2f = O.to_f64(inp["W2"]) if cfg.target_from_draft else None
    for r in range(R):
        if cfg.target_from_draft and r in req:
            zd = O.draft_logits_all(inp["U"], inp["W1"], W2f, inp["anchors"][[r]], tokens[[r]], [r])[0]
            base = zd.astype(np.float32)
        else:
            base = O.to_f64(inp["U"][r]).astype(np.float32)
        T[r] = synth.target_rows(cfg, r, base, inp["Ub"][r])
    return T


def compare_draft(od, tokens, lse, logq, requests=None):
    """Compare a GPU draft (numpy arrays [R, gamma]) with the oracle's result
    ``od`` for ``requests`` (rows of od in that order).  Returns (n_compared,
    n_ties); raises AssertionError on a hard mismatch."""
    req = od["requests"] if requests is None else requests
    compared = ties = 0
    for i, r in enumerate(req):
        for k in range(od["tokens"].shape[1]):
            if tokens[r, k] != od["tokens"][i, k]:
                m = od["margin"][i, k]
                assert m < TIE, (f"draft token mismatch r={r} k={k+1}: gpu {tokens[r, k]} "
                                 f"oracle {od['tokens'][i, k]} margin {m:.3e}")
                ties += 1
                log(f"near-tie draft r={r} k={k+1} margin={m:.2e}")
                break
            compared += 1
            _track("max_lse_d_err", abs(lse[r, k] - od["lse"][i, k]))
            np.testing.assert_allclose(lse[r, k], od["lse"][i, k], rtol=RTOL, atol=ATOL,
                                       err_msg=f"lse r={r} k={k+1}")
            # logq = ln p^d(x): p^d within RTOL relative is logq within RTOL absolute
            np.testing.assert_allclose(logq[r, k], od["logq"][i, k], rtol=0, atol=RTOL,
                                       err_msg=f"logq r={r} k={k+1}")
            np.testing.assert_allclose(np.exp(logq[r, k]), np.exp(od["logq"][i, k]), rtol=RTOL,
                                       atol=ATOL, err_msg=f"p^d(x) r={r} k={k+1}")
    STATS["draws"] += compared + ties
    STATS["ties"] += ties
    return compared, ties


def compare_verify(ov, g, requests=None, rho=None):
    """Compare GPU verify outputs (numpy dict) with the oracle's ``ov`` for its
    requests.  ``rho`` = (T, tokens, logq_in, logq_oracle) also tracks how far
    the GPU's acceptance log-ratio (T[x] - lse_t) - logq_in is from the
    oracle's (T[x] - lse_t) - logq_oracle (T stored target logits [R, gamma+1,
    V], tokens and logq_in [R, gamma] by request id, logq_oracle [n, gamma] in
    ``ov``'s row order).  Returns (n_requests_compared, n_ties)."""
    req = ov["requests"] if requests is None else requests
    ties = decisions = 0
    gamma = ov["cstar"].shape[1]
    for i, r in enumerate(req):
        if rho is not None and g.get("lse_t") is not None:
            T, tokens, logq_in, logq_or = rho
            for k in range(int(np.sum(ov["accept_mask"][i] != 255))):
                x = int(tokens[r, k])
                tx = float(O.to_f64(T[r, k, x:x + 1])[0])
                rho_g = (tx - g["lse_t"][r, k]) - logq_in[r, k]
                rho_o = (tx - ov["lse_t"][i, k]) - logq_or[i, k]
                _track("max_rho_err", abs(rho_g - rho_o))
        oc, gc = ov["cstar"][i], g["cstar"][r]
        assert np.array_equal(np.isnan(oc), np.isnan(gc)), f"c* NaN pattern r={r}"
        fin = ~np.isnan(oc)
        np.testing.assert_allclose(gc[fin], oc[fin], rtol=RTOL, atol=ATOL, err_msg=f"c* r={r}")
        if g.get("lse_t") is not None:
            olt, glt = ov["lse_t"][i], g["lse_t"][r]
            fin = ~np.isnan(olt)
            if fin.any():
                _track("max_lse_t_err", np.max(np.abs(glt[fin] - olt[fin])))
            np.testing.assert_allclose(glt[fin], olt[fin], rtol=RTOL, atol=ATOL, err_msg=f"lse_t r={r}")
        tie_here = False
        for k in range(gamma):
            om, gm = ov["accept_mask"][i, k], g["accept_mask"][r, k]
            if om != gm:
                m = ov["acc_margin"][i, k]
                assert m < TIE, f"accept mismatch r={r} k={k+1}: gpu {gm} oracle {om} margin {m:.3e}"
                log(f"near-tie accept r={r} k={k+1} margin={m:.2e}")
                tie_here = True
                ties += 1
                break
            if om == 255:
                break
            decisions += 1
            if om != 1:
                break
        if tie_here:
            continue
        assert g["n_accept"][r] == ov["n_accept"][i], f"n_accept r={r}"
        if g["out_token"][r] != ov["out_token"][i]:
            m = ov["out_margin"][i]
            assert m < TIE, (f"out_token mismatch r={r}: gpu {g['out_token'][r]} oracle "
                             f"{ov['out_token'][i]} margin {m:.3e}")
            log(f"near-tie final draw r={r} margin={m:.2e}")
            ties += 1
        else:
            decisions += 1
    STATS["draws"] += decisions + ties
    STATS["ties"] += ties
    return len(req), ties


def compare_logpd(logpd_g, U, W1, W2f, anchors, tok_g, od, requests=None, k_range=None):
    """Element-by-element check of the draft's log p^d output [R, gamma, V]
    against the oracle: p^d within RTOL relative / ATOL absolute, for every
    (request, position) whose earlier drafted tokens equal the oracle's (the
    rows are conditioned on them).  ``od`` is the oracle draft of ``requests``
    (rows in that order).  Returns the number of rows compared."""
    req = od["requests"] if requests is None else requests
    gamma = od["tokens"].shape[1]
    rows = 0
    for k in (range(1, gamma + 1) if k_range is None else k_range):
        same = np.array([np.array_equal(tok_g[r, :k - 1], od["tokens"][i, :k - 1])
                         for i, r in enumerate(req)])
        sel = np.asarray(req)[same]
        if sel.size == 0:
            continue
        prev = anchors[sel] if k == 1 else od["tokens"][same, k - 2]
        z = O.draft_logits(U[sel, k - 1, :], W1, W2f, prev)
        lpd_o = z - od["lse"][same, k - 1][:, None]
        lpd_g = logpd_g[sel, k - 1, :].astype(np.float64)
        _track("max_logpd_err", np.max(np.abs(lpd_g - lpd_o)))
        np.testing.assert_allclose(np.exp(lpd_g), np.exp(lpd_o), rtol=RTOL, atol=ATOL,
                                   err_msg=f"p^d at position {k}")
        STATS["logpd_values"] += lpd_g.size
        rows += sel.size
    return rows


def compare_schedule(os_, a_g, g):
    """Compare GPU scheduler outputs with the oracle's (a bit-exact)."""
    np.testing.assert_array_equal(a_g, os_["a"])
    if not np.array_equal(g["lengths"], os_["lengths"]):
        assert os_["stop_gap"] < TIE, f"schedule lengths differ, stop gap {os_['stop_gap']:.3e}"
        log(f"near-tie schedule stop gap={os_['stop_gap']:.2e}")
        return 1
    np.testing.assert_allclose(g["stats"], os_["stats"], rtol=1e-12, atol=0)
    np.testing.assert_allclose(g["theta_path"], os_["theta_path"], rtol=1e-12, atol=0, equal_nan=True)
    return 0

"""GPU parity at the workloads' full sizes (C2 Qwen3-4B-shaped, C3 high
concurrency, C4 large vocabulary, C5 full scheduled round), in the launch
configuration the benchmark times: the whole batch goes through the C ABI and
every request is compared with the oracle (a request's draft, verification and
confidence depend on its own inputs only; the scheduler, which couples
requests, is compared on the whole batch).  At C2 and C3 the draft runs a
second time with its log p^d output, which is compared with the oracle element
by element.

Target logits are built from the ORACLE's draft logits (draft logits + noise,
the workloads' recipe), so no oracle input comes from the HIP path.  A request
whose GPU draft parted from the oracle's at a logged near-tie is left out of
the verify comparison (its targets follow the oracle's tokens).
"""
import numpy as np
import pytest

from parity_util import (compare_draft, compare_logpd, compare_schedule, compare_verify, log,
                         to_dev)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from draft_sampling_verification_w1_amd import dspark
    dspark.lib()
    return dspark


def _targets(cfg, inp, od_tokens, synth, O):
    """T [R, gamma+1, V] in storage type: the oracle's draft logits + noise
    (one fp64 product per position over the whole batch)."""
    R, g, V = cfg.R, cfg.gamma, cfg.V
    W2f = O.to_f64(inp["W2"])
    base = np.empty((R, g, V), np.float32)
    for k in range(1, g + 1):
        prev = inp["anchors"] if k == 1 else od_tokens[:, k - 2]
        base[:, k - 1, :] = O.draft_logits(inp["U"][:, k - 1, :], inp["W1"], W2f, prev)
    T = np.empty((R, g + 1, V), np.uint16)
    for r in range(R):
        T[r] = synth.target_rows(cfg, r, base[r], inp["Ub"][r])
    return T


def _full_round(dev, name, with_confidence=False, check_logpd=False):
    import time
    import torch
    from oracle import oracle as O
    from draft_sampling_verification_w1_amd import synth
    cfg = synth.CONFIGS[name]
    t0 = time.time()
    W1, W2 = synth.weights(cfg)
    U, Ub = synth.backbone(cfg)
    inp = {"W1": W1, "W2": W2, "U": U, "Ub": Ub, "anchors": synth.anchors(cfg)}
    log(f"full size {name}: R={cfg.R} gamma={cfg.gamma} V={cfg.V}; inputs in {time.time() - t0:.1f}s")

    dU, dW1, dA = to_dev(U), to_dev(W1), to_dev(inp["anchors"])
    W2p = dev.pack_w2(to_dev(W2), cfg.V)
    tok, lse, logq = dev.draft_step(dU, dW1, W2p, dA, cfg.seed)
    torch.cuda.synchronize()
    tok_h, lse_h, logq_h = tok.cpu().numpy(), lse.cpu().numpy(), logq.cpu().numpy()
    t0 = time.time()
    od = O.draft(U, W1, W2, inp["anchors"], cfg.seed)
    n, ties = compare_draft(od, tok_h, lse_h, logq_h)
    log(f"  draft: {n} positions compared (every request), {ties} near-ties; oracle "
        f"{time.time() - t0:.1f}s")
    assert np.all((tok_h >= 0) & (tok_h < cfg.V))

    if check_logpd:
        lp = torch.empty((cfg.R, cfg.gamma, cfg.V), dtype=torch.float32, device="cuda")
        tok2 = dev.draft_step(dU, dW1, W2p, dA, cfg.seed, logpd=lp)[0]
        torch.cuda.synchronize()
        assert torch.equal(tok2, tok), "the draft with the log p^d output drew other tokens"
        t0 = time.time()
        rows = compare_logpd(lp.cpu().numpy(), U, W1, O.to_f64(W2), inp["anchors"], tok_h, od)
        del lp
        log(f"  log p^d: {rows} rows x {cfg.V} compared element by element in "
            f"{time.time() - t0:.1f}s")

    lengths = None
    if with_confidence:
        # confidence head on every position from the drafted tokens, then the
        # scheduler on the whole batch
        h, w = synth.confidence_inputs(cfg)
        temps = synth.sts_temperatures(cfg)
        gc = dev.confidence(to_dev(h), to_dev(w), to_dev(temps), dW1, dA, tok).cpu().numpy()
        oc = O.confidence(h, w, temps, W1, inp["anchors"], tok_h)
        ulp = np.abs(gc.view(np.int32).astype(np.int64) - oc.view(np.int32).astype(np.int64))
        assert ulp.max() <= 1, f"confidence differs by {ulp.max()} ulp"
        a = O.prefix_products(oc)
        sps = synth.sps_table(cfg)
        os_ = O.schedule(a, sps)
        os_["a"] = a
        gs = dev.schedule(to_dev(oc), to_dev(sps))
        torch.cuda.synchronize()
        compare_schedule(os_, gs["a"].cpu().numpy(), {k: v.cpu().numpy() for k, v in gs.items() if k != "a"})
        lengths = os_["lengths"]
        log(f"  confidence + schedule: n_sel {int(os_['stats'][3])}, B {int(os_['stats'][0])}, "
            f"mean length {lengths.mean():.2f}")

    t0 = time.time()
    T = _targets(cfg, inp, od["tokens"], synth, O)
    log(f"  targets in {time.time() - t0:.1f}s")
    g = dev.verify(dU, dW1, W2p, dA, tok, lse, logq, to_dev(T),
                   None if lengths is None else to_dev(lengths), cfg.seed)
    torch.cuda.synchronize()
    gn = {k: (v.cpu().numpy() if v is not None else None) for k, v in g.items()}
    same = np.array([np.array_equal(tok_h[r], od["tokens"][r]) for r in range(cfg.R)])
    req = np.nonzero(same)[0].astype(np.int32)
    t0 = time.time()
    ov = O.verify(U, W1, W2, inp["anchors"], tok_h, T, lengths, cfg.seed, requests=req, chunk=32)
    n, ties = compare_verify(ov, gn, requests=req, rho=(T, tok_h, logq_h, od["logq"][req]))
    log(f"  verify: {n} of {cfg.R} requests compared, {ties} near-ties; oracle "
        f"{time.time() - t0:.1f}s; mean accepted {ov['n_accept'].mean():.3f}")
    assert n >= cfg.R - 2
    # every request: lengths and token ranges are consistent
    L = np.full(cfg.R, cfg.gamma) if lengths is None else lengths
    assert np.all((gn["n_accept"] >= 0) & (gn["n_accept"] <= L))
    assert np.all((gn["out_token"] >= 0) & (gn["out_token"] < cfg.V))
    fin = ~np.isnan(gn["cstar"])
    assert np.array_equal(fin, np.arange(cfg.gamma)[None, :] < L[:, None])
    assert np.all((gn["cstar"][fin] >= -1e-6) & (gn["cstar"][fin] <= 1 + 1e-6))

    if not with_confidence:
        # scheduler on the round's c* (whole batch, c* from the GPU)
        c = np.nan_to_num(gn["cstar"], nan=0.0).astype(np.float32)
        a = O.prefix_products(c)
        sps = synth.sps_table(cfg)
        os_ = O.schedule(a, sps)
        os_["a"] = a
        gs = dev.schedule(to_dev(c), to_dev(sps))
        torch.cuda.synchronize()
        compare_schedule(os_, gs["a"].cpu().numpy(), {k: v.cpu().numpy() for k, v in gs.items() if k != "a"})
        log(f"  schedule on c*: n_sel {int(os_['stats'][3])}, B {int(os_['stats'][0])}")


def test_full_size_qwen3_4b(dev):
    _full_round(dev, "qwen3_4b", check_logpd=True)


def test_full_size_high_concurrency(dev):
    _full_round(dev, "high_concurrency", check_logpd=True)


def test_full_size_large_vocab(dev):
    _full_round(dev, "large_vocab")


def test_full_size_scheduled_round(dev):
    _full_round(dev, "full_round", with_confidence=True)


def test_maximum_batch(dev):
    """The library's batch limits, R = 65,536 requests and R * gamma = 2^20
    positions, at a two-tile vocabulary (V = 40): draft and verify of the
    whole batch against the oracle, compared with array operations (the
    scheduler's own limit, R * gamma <= 16,384, is covered above)."""
    import time
    import torch
    from oracle import oracle as O
    from draft_sampling_verification_w1_amd import synth
    from parity_util import RTOL, ATOL, TIE, STATS
    cfg = synth.scaled(synth.CONFIGS["high_concurrency"], name="max_batch", R=65536, gamma=16, V=40,
                       n_sps=65536 * 17)
    R, g, V = cfg.R, cfg.gamma, cfg.V
    t0 = time.time()
    W1, W2 = synth.weights(cfg)
    U, Ub = synth.backbone(cfg)
    A = synth.anchors(cfg)
    log(f"maximum batch: R={R} gamma={g} V={V}; inputs in {time.time() - t0:.1f}s")

    dU, dW1, dA = to_dev(U), to_dev(W1), to_dev(A)
    W2p = dev.pack_w2(to_dev(W2), V)
    tok, lse, logq = dev.draft_step(dU, dW1, W2p, dA, cfg.seed)
    torch.cuda.synchronize()
    tok_h, lse_h, logq_h = tok.cpu().numpy(), lse.cpu().numpy(), logq.cpu().numpy()
    od = O.draft(U, W1, W2, A, cfg.seed)
    # a request is compared up to its first differing token, which must be
    # an oracle near-tie (the later positions then condition on other tokens)
    diff = tok_h != od["tokens"]
    first = np.where(diff.any(axis=1), diff.argmax(axis=1), g)
    tied = np.nonzero(first < g)[0]
    assert np.all(od["margin"][tied, first[tied]] < TIE), "draft token mismatch beyond a near-tie"
    upto = np.arange(g)[None, :] < first[:, None]
    np.testing.assert_allclose(lse_h[upto], od["lse"][upto], rtol=RTOL, atol=ATOL)
    np.testing.assert_allclose(logq_h[upto], od["logq"][upto], rtol=0, atol=RTOL)
    draws = int(upto.sum()) + tied.size
    STATS["draws"] += draws
    STATS["ties"] += tied.size
    assert tied.size <= 1e-4 * draws
    log(f"  draft: {draws} positions compared, {tied.size} near-ties")

    # targets from the oracle's draft logits (the workload's recipe)
    W2f = O.to_f64(W2)
    base = np.empty((R, g, V), np.float32)
    for k in range(1, g + 1):
        prev = A if k == 1 else od["tokens"][:, k - 2]
        base[:, k - 1, :] = O.draft_logits(U[:, k - 1, :], W1, W2f, prev)
    T = np.empty((R, g + 1, V), np.uint16)
    for r in range(R):
        T[r] = synth.target_rows(cfg, r, base[r], Ub[r])
    gv = dev.verify(dU, dW1, W2p, dA, tok, lse, logq, to_dev(T), None, cfg.seed)
    torch.cuda.synchronize()
    gn = {k: (v.cpu().numpy() if v is not None else None) for k, v in gv.items()}
    req = np.nonzero(first == g)[0].astype(np.int32)
    ov = O.verify(U, W1, W2, A, tok_h, T, None, cfg.seed, requests=req, chunk=4096)
    np.testing.assert_allclose(gn["cstar"][req], ov["cstar"], rtol=RTOL, atol=ATOL)
    np.testing.assert_allclose(gn["lse_t"][req], ov["lse_t"], rtol=RTOL, atol=ATOL)
    # acceptance: a differing decision must be an oracle near-tie
    am = gn["accept_mask"][req] != ov["accept_mask"]
    mism = np.nonzero(am.any(axis=1))[0]
    k0 = am.argmax(axis=1)
    assert np.all(ov["acc_margin"][mism, k0[mism]] < TIE), "accept decision differs beyond a near-tie"
    same = np.ones(req.size, bool)
    same[mism] = False
    assert np.array_equal(gn["n_accept"][req][same], ov["n_accept"][same])
    tok_diff = np.nonzero(same & (gn["out_token"][req] != ov["out_token"]))[0]
    assert np.all(ov["out_margin"][tok_diff] < TIE), "corrective / bonus token differs beyond a near-tie"
    ties = mism.size + tok_diff.size
    STATS["draws"] += req.size
    STATS["ties"] += ties
    assert ties <= 1e-4 * req.size * g
    log(f"  verify: {req.size} requests compared, {ties} near-ties; mean accepted "
        f"{ov['n_accept'].mean():.3f}")

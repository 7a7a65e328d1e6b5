"""GPU parity of multi-round decoding: the DecodeLoop (draft + verify through
the C ABI, anchors handed over on the device, per-round Philox keys) against
the oracle's loop over the same per-round inputs.  A request whose chain
parts from the oracle's at an allowed near-tie (oracle margin below 1e-6) is
compared no further."""
import numpy as np
import pytest

from parity_util import compare_draft, compare_verify, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from draft_sampling_verification_w1_amd import dspark
    dspark.lib()
    return dspark


def _rows(d, idx):
    return {k: (v[idx] if isinstance(v, np.ndarray) and v.ndim >= 1 and v.shape[0] == len(d["requests"]) else v)
            for k, v in d.items()}


@pytest.mark.parametrize("name,R,gamma,V,rounds", [
    ("high_concurrency", 16, 4, 3000, 5),
    ("tiny", 4, 8, 4096, 3),
    ("full_round", 37, 3, 2049, 3),
])
def test_decode_loop(dev, name, R, gamma, V, rounds):
    import torch
    from oracle import oracle as O
    from draft_sampling_verification_w1_amd import synth
    from draft_sampling_verification_w1_amd.decode import DecodeLoop, round_seed
    import test_oracle_decode as D
    cfg = synth.scaled(synth.CONFIGS[name], name="loop", R=R, gamma=gamma, V=V,
                       n_sps=R * (gamma + 1))
    log(f"case decode loop {name} R={R} gamma={gamma} V={V} rounds={rounds}")
    res, W1, W2 = D._loop(O, cfg, rounds)
    loop = DecodeLoop(to_dev(W1), dev.pack_w2(to_dev(W2), cfg.V), to_dev(synth.anchors(cfg)),
                      cfg.seed, gamma)
    live = np.arange(R)
    for t in range(rounds):
        assert round_seed(cfg.seed, t) == res[t]["key"]
        g = loop.round(to_dev(res[t]["U"]), lambda tt, tok: to_dev(res[tt]["T"]))
        torch.cuda.synchronize()
        gn = {k: (v.cpu().numpy() if torch.is_tensor(v) else v) for k, v in g.items()}
        od, ov = _rows(res[t]["draft"], live), _rows(res[t]["verify"], live)
        np.testing.assert_array_equal(gn["anchors"][live], res[t]["anchors"][live])
        n, dt = compare_draft(od, gn["tokens"], gn["lse"], gn["logq"], requests=live)
        _, vt = compare_verify(ov, gn, requests=live)
        same = (gn["out_token"][live] == ov["out_token"]) & np.all(gn["tokens"][live] == od["tokens"], axis=1)
        if not same.all():
            log(f"  round {t}: {int((~same).sum())} request(s) left the comparison at a near-tie")
        live = live[same]
        tau = gn["n_accept"] + 1
        log(f"  round {t}: {n} positions compared, mean tau {tau.mean():.2f}")
    assert live.size > 0

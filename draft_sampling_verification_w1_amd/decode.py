"""Multi-round decoding over the C ABI: each round drafts a block of gamma
positions from the requests' anchors, verifies it against the target logits
and emits the accepted prefix plus one corrective or bonus token; that last
token is the next round's anchor.  Summary page §요약 (a drafted block is
verified by rejection sampling, which keeps the target distribution), §3
(a round's accepted length tau counts the bonus token; per-token latency
L = (T_draft + T_verify) / tau) and §3.1 (a block is drafted from the anchor).

Round t draws its random numbers with the Philox key seed + t * 2^32 (the
round index in the key's high word), so round 0 is the single-round call and
different rounds use independent streams.  The anchors are handed from one
round to the next on the device (two alternating buffers, no host copy).
Argument marshalling only: every step runs in the HIP library.
"""
from __future__ import annotations

import torch

from . import dspark

ROUND_KEY_STRIDE = 1 << 32


def round_seed(seed: int, t: int) -> int:
    """Philox key of round t: the round index added to the key's high word."""
    return (int(seed) + int(t) * ROUND_KEY_STRIDE) & ((1 << 64) - 1)


class DecodeLoop:
    """Rounds of draft + verify (+ Algorithm 1 on the round's c*, when an SPS
    table is given) with the anchors carried on the device.

    W1 [V, 256] and W2p (packed) stay fixed; each round takes its backbone
    logits U [R, gamma, V] and a callable that returns the target logits
    T [R, gamma + 1, V] for the drafted tokens (the target model's verify
    forward pass)."""

    def __init__(self, W1, W2p, anchors, seed: int, gamma: int, sps=None):
        R = anchors.numel()
        V = W1.shape[0]
        dev = W1.device
        self.W1, self.W2p, self.seed, self.gamma, self.sps = W1, W2p, int(seed), gamma, sps
        self.t = 0
        self._anchors = [anchors.clone(), torch.empty_like(anchors)]
        self.ws = dspark.workspace(dspark.problem(R, gamma, V, W1.dtype, seed), dev)
        self.d_out = (torch.empty((R, gamma), dtype=torch.int32, device=dev),
                      torch.empty((R, gamma), dtype=torch.float64, device=dev),
                      torch.empty((R, gamma), dtype=torch.float64, device=dev))
        self.v_out = {"cstar": torch.empty((R, gamma), dtype=torch.float32, device=dev),
                      "n_accept": torch.empty(R, dtype=torch.int32, device=dev),
                      "out_token": None,
                      "accept_mask": torch.empty((R, gamma), dtype=torch.uint8, device=dev),
                      "lse_t": None}
        self.s_out = {"a": torch.empty((R, gamma), dtype=torch.float32, device=dev),
                      "lengths": torch.empty(R, dtype=torch.int32, device=dev),
                      "stats": torch.empty(4, dtype=torch.float64, device=dev),
                      "theta_path": None}

    @property
    def anchors(self):
        """Anchors of the next round (device int32 [R])."""
        return self._anchors[self.t % 2]

    def round(self, U, target_fn):
        """One round; returns a dict of device tensors: tokens, lse, logq,
        cstar, n_accept, out_token (= the next anchors), accept_mask and, with
        an SPS table, the scheduler's a, lengths and stats."""
        seed_t = round_seed(self.seed, self.t)
        anchors = self._anchors[self.t % 2]
        nxt = self._anchors[(self.t + 1) % 2]
        tok, lse, logq = dspark.draft_step(U, self.W1, self.W2p, anchors, seed_t, ws=self.ws,
                                           out=self.d_out)
        T = target_fn(self.t, tok)
        self.v_out["out_token"] = nxt
        v = dspark.verify(U, self.W1, self.W2p, anchors, tok, lse, logq, T, None, seed_t,
                          ws=self.ws, out=self.v_out)
        res = {"tokens": tok, "lse": lse, "logq": logq, "cstar": v["cstar"],
               "n_accept": v["n_accept"], "out_token": nxt, "accept_mask": v["accept_mask"],
               "anchors": anchors, "seed": seed_t}
        if self.sps is not None:
            s = dspark.schedule(v["cstar"], self.sps, out=self.s_out, with_path=False)
            res.update({"a": s["a"], "lengths": s["lengths"], "stats": s["stats"]})
        self.t += 1
        return res

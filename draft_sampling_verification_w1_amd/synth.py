"""Seeded synthetic inputs for the DSpark draft-and-verify hot path.

This module only draws random inputs and rounds them to their storage type.
It holds none of the method's arithmetic (no contraction, softmax, sampling or
scheduling), and is the one module that both the HIP path and the CPU oracle
use.  Every array comes from NumPy's PCG64 seeded by a SeedSequence of
(config seed, purpose tag, request index), so any request's inputs can be
regenerated alone and in any order.

Storage: bfloat16 tensors are numpy uint16 arrays holding bf16 bit patterns
(fp32 draws rounded to nearest even); fp32 tensors are numpy float32 arrays.

Workload shapes follow the pages' vocabularies and block sizes (the summary
page's §4.1 and §5.1): Qwen3's 151,936-token vocabulary, a DeepSeek-scale
~10^5 vocabulary (129,280), a 262,144-token large vocabulary, rank-256 Markov
head factors.  The benchmark suites the pages measure on are not used; these
draws stand in for their logits.
"""
from __future__ import annotations

import dataclasses

import numpy as np

# purpose tags for SeedSequence([seed, tag, index])
_TAG_W1, _TAG_W2, _TAG_ANCHOR, _TAG_U, _TAG_BOOST, _TAG_BONUS, _TAG_NOISE = 1, 2, 3, 4, 5, 6, 7
_TAG_H, _TAG_W, _TAG_SCHED = 8, 9, 10


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    R: int
    gamma: int
    V: int
    rank: int
    dtype: str                 # "f32" or "bf16"
    seed: int
    u_sigma: float             # std of backbone logits U
    w_sigma: float             # std of W1, W2 entries
    zipf_boost: float          # +boost on one Zipf-ranked token per (r,k); 0 = none
    target_from_draft: bool    # T = draft logits + noise (else U + noise)
    noise: str                 # noise-sigma rule name
    sps: str                   # SPS table rule name
    n_sps: int
    confidence_H: int = 0      # >0: confidence head inputs exist (full scheduled round)

    @property
    def positions(self) -> int:
        return self.R * self.gamma

    def noise_sigma(self, k: int) -> float:
        """Target-noise std at block position k (1-based; k = gamma+1 is the bonus row)."""
        if self.noise == "unit":
            return 1.0
        if self.noise == "rising":       # 0.7 at k = 1, rising with k
            return 0.7 + 0.05 * (k - 1)
        if self.noise == "decaying":     # sigma_k = 0.3 + 0.1 k
            return 0.3 + 0.1 * k
        raise ValueError(self.noise)


CONFIGS = {
    "tiny": Config("tiny", R=4, gamma=8, V=4096, rank=256, dtype="f32", seed=0, u_sigma=3.0,
                   w_sigma=0.05, zipf_boost=0.0, target_from_draft=False, noise="unit",
                   sps="tiny", n_sps=64),
    "qwen3_4b": Config("qwen3_4b", R=32, gamma=16, V=151936, rank=256, dtype="bf16", seed=1,
                       u_sigma=4.0, w_sigma=0.02, zipf_boost=8.0, target_from_draft=True,
                       noise="rising", sps="knee512", n_sps=32 * 17),
    "high_concurrency": Config("high_concurrency", R=256, gamma=16, V=151936, rank=256,
                               dtype="bf16", seed=2, u_sigma=4.0, w_sigma=0.02, zipf_boost=8.0,
                               target_from_draft=True, noise="decaying", sps="knee512",
                               n_sps=4352),
    "large_vocab": Config("large_vocab", R=128, gamma=16, V=262144, rank=256, dtype="bf16",
                          seed=3, u_sigma=3.0, w_sigma=0.05, zipf_boost=0.0,
                          target_from_draft=True, noise="unit", sps="knee512",
                          n_sps=128 * 17),
    "full_round": Config("full_round", R=512, gamma=16, V=129280, rank=256, dtype="bf16", seed=4,
                         u_sigma=4.0, w_sigma=0.02, zipf_boost=8.0, target_from_draft=True,
                         noise="decaying", sps="knee2R", n_sps=8704, confidence_H=4096),
}


def scaled(cfg: Config, **changes) -> Config:
    """A copy of a config with some fields replaced (smaller shapes for tests)."""
    return dataclasses.replace(cfg, **changes)


def _rng(cfg: Config, tag: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg.seed, tag, index]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to bfloat16 (nearest, ties to even); finite inputs."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((b + (0x7FFF + ((b >> 16) & 1))) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(cfg: Config, x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, np.float32)
    return f32_to_bf16_bits(x) if cfg.dtype == "bf16" else x


def weights(cfg: Config):
    """Markov-head factors W1 [V, rank] and W2 [rank, V] in storage type."""
    W1 = _rng(cfg, _TAG_W1).standard_normal((cfg.V, cfg.rank), dtype=np.float32) * np.float32(cfg.w_sigma)
    W2 = _rng(cfg, _TAG_W2).standard_normal((cfg.rank, cfg.V), dtype=np.float32) * np.float32(cfg.w_sigma)
    return _store(cfg, W1), _store(cfg, W2)


def anchors(cfg: Config) -> np.ndarray:
    """Anchor token per request, uniform over the vocabulary."""
    return _rng(cfg, _TAG_ANCHOR).integers(0, cfg.V, size=cfg.R, dtype=np.int64).astype(np.int32)


def _zipf_ids(rng: np.random.Generator, n: int, V: int, a: float = 1.1) -> np.ndarray:
    """Token ids t-1 with rank t ~ Zipf(a) truncated to [1, V]."""
    p = np.arange(1, V + 1, dtype=np.float64) ** (-a)
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    return np.searchsorted(cdf, rng.random(n), side="right").clip(0, V - 1).astype(np.int64)


def backbone_row_f32(cfg: Config, r: int) -> np.ndarray:
    """Backbone logits U[r] as fp32 draws [gamma + 1, V]; row gamma is the extra
    row U' that seeds the bonus target row."""
    rng = _rng(cfg, _TAG_U, r)
    U = rng.standard_normal((cfg.gamma + 1, cfg.V), dtype=np.float32) * np.float32(cfg.u_sigma)
    if cfg.zipf_boost:
        ids = _zipf_ids(_rng(cfg, _TAG_BOOST, r), cfg.gamma + 1, cfg.V)
        U[np.arange(cfg.gamma + 1), ids] += np.float32(cfg.zipf_boost)
    return U


def backbone(cfg: Config, requests=None):
    """U [n, gamma, V] and the bonus base rows U' [n, V], in storage type."""
    req = range(cfg.R) if requests is None else requests
    req = list(req)
    dt = np.uint16 if cfg.dtype == "bf16" else np.float32
    U = np.empty((len(req), cfg.gamma, cfg.V), dt)
    Ub = np.empty((len(req), cfg.V), dt)
    for i, r in enumerate(req):
        full = _store(cfg, backbone_row_f32(cfg, r))
        U[i] = full[:cfg.gamma]
        Ub[i] = full[cfg.gamma]
    return U, Ub


def target_noise(cfg: Config, r: int) -> np.ndarray:
    """Target noise for request r: [gamma + 1, V] fp32, row k-1 with std sigma_k."""
    rng = _rng(cfg, _TAG_NOISE, r)
    n = rng.standard_normal((cfg.gamma + 1, cfg.V), dtype=np.float32)
    sig = np.array([cfg.noise_sigma(k) for k in range(1, cfg.gamma + 2)], np.float32)
    return n * sig[:, None]


def target_rows(cfg: Config, r: int, base_f32: np.ndarray, bonus_base: np.ndarray) -> np.ndarray:
    """Target logits T[r] = storage(base + noise) for rows 1..gamma, and
    storage(U' + noise) for the bonus row gamma+1.

    base_f32: [gamma, V] fp32 -- the request's draft logits where the config's
    target is built from them (the caller computes those), else its U rows.
    bonus_base: [V] stored U' row."""
    noise = target_noise(cfg, r)
    out = np.empty((cfg.gamma + 1, cfg.V), np.float32)
    out[:cfg.gamma] = np.asarray(base_f32, np.float32) + noise[:cfg.gamma]
    bb = bf16_bits_to_f32(bonus_base) if cfg.dtype == "bf16" else np.asarray(bonus_base, np.float32)
    out[cfg.gamma] = bb + noise[cfg.gamma]
    return _store(cfg, out)


def sps_table(cfg: Config) -> np.ndarray:
    """Engine step-rate table SPS(B) for B = 1..n_sps (entry B-1), fp32."""
    B = np.arange(1, cfg.n_sps + 1, dtype=np.float64)
    if cfg.sps == "tiny":
        s = 1000.0 / (1.0 + 0.01 * B)
    elif cfg.sps == "knee512":       # flat to B = 512, then ~1/B
        s = 1000.0 * np.minimum(1.0, 512.0 / B)
    elif cfg.sps == "knee2R":        # flat to B = 2R, then ~1/B
        s = 1000.0 * np.minimum(1.0, 2.0 * cfg.R / B)
    else:
        raise ValueError(cfg.sps)
    return s.astype(np.float32)


def sts_temperatures(cfg: Config) -> np.ndarray:
    """Per-position STS temperatures spanning [0.8, 1.5] linearly."""
    g = cfg.gamma
    k = np.arange(1, g + 1, dtype=np.float64)
    t = 0.8 + 0.7 * (k - 1) / max(g - 1, 1)
    return t.astype(np.float32)


def confidence_inputs(cfg: Config, requests=None):
    """Backbone states h [n, gamma, H] (bf16 bits) and head weights w [H + rank] fp32."""
    H = cfg.confidence_H
    req = list(range(cfg.R) if requests is None else requests)
    h = np.empty((len(req), cfg.gamma, H), np.uint16)
    for i, r in enumerate(req):
        h[i] = f32_to_bf16_bits(_rng(cfg, _TAG_H, r).standard_normal((cfg.gamma, H), dtype=np.float32))
    w = (_rng(cfg, _TAG_W).standard_normal(H + cfg.rank, dtype=np.float32) * np.float32(0.01))
    return h, w


def survival_inputs(cfg: Config, index: int = 0) -> np.ndarray:
    """Stand-alone per-position confidences c [R, gamma] in (0, 1], for
    exercising the scheduler on its own (beta-distributed, decaying with k)."""
    rng = _rng(cfg, _TAG_SCHED, index)
    k = np.arange(1, cfg.gamma + 1)[None, :]
    mean = 0.95 - 0.5 * (k - 1) / max(cfg.gamma - 1, 1)
    c = rng.beta(20.0 * mean, 20.0 * (1.0 - mean), size=(cfg.R, cfg.gamma))
    return c.astype(np.float32)

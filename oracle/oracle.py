"""Plain fp64 CPU oracle for the DSpark per-round draft-and-verify hot path.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code with
the HIP library; the two meet only through the seeded input generators.

Pages cited (titles as published):
  [P1] "DSpark: Confidence-Scheduled Speculative Decoding with Semi-Autoregressive
       Generation 요약 설명" (summary page)
  [P2] "DSpark: Confidence-Scheduled Speculative Decoding with Semi-Autoregressive
       Generation" (notes page, "DSpark 핵심 기술")

The per-element work (random numbers, softmax, Gumbel-max, c*, acceptance,
residual and bonus draws, Algorithm 1) is in ``dspark_oracle.c`` as straight
fp64 loops.  This module only marshals arrays and forms the logits
z = U_k + W1[x_{k-1}] W2 with a library fp64 matrix product ([P1 §3.1]:
B = W1 W2 with rank r; the head conditions on the previous token).

Parity pins for every function live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dspark_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

#: entries per block of the two-level Gumbel-max draws
SAMPLE_BLOCK = 32

_f64p = ctypes.POINTER(ctypes.c_double)
_f32p = ctypes.POINTER(ctypes.c_float)
_i32p = ctypes.POINTER(ctypes.c_int32)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i64p = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (-O2, no fast-math, OpenMP over rows)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_philox4x32_10.argtypes = [ctypes.c_uint32, ctypes.c_uint32, _u32p, _u32p]
        L.oracle_word.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                  ctypes.c_uint32, ctypes.c_uint32]
        L.oracle_word.restype = ctypes.c_uint32
        L.oracle_words.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                   ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int64, _u32p]
        L.oracle_uniform.argtypes = [ctypes.c_uint32]
        L.oracle_uniform.restype = ctypes.c_double
        L.oracle_gumbel.argtypes = [ctypes.c_uint32]
        L.oracle_gumbel.restype = ctypes.c_double
        L.oracle_logsumexp.argtypes = [ctypes.c_int64, _f64p]
        L.oracle_logsumexp.restype = ctypes.c_double
        L.oracle_gumbel_argmax.argtypes = [ctypes.c_int64, _f64p, _f64p, _f64p]
        L.oracle_gumbel_argmax.restype = ctypes.c_int64
        L.oracle_two_level_draw.argtypes = [ctypes.c_int64, _f64p, ctypes.c_int64,
                                            ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                            ctypes.c_uint32, ctypes.c_uint32, _f64p]
        L.oracle_two_level_draw.restype = ctypes.c_int64
        L.oracle_accept.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double]
        L.oracle_accept.restype = ctypes.c_int
        L.oracle_residual_logw.argtypes = [ctypes.c_int64, _f64p, _f64p, _f64p]
        L.oracle_residual_logw.restype = ctypes.c_int64
        L.oracle_cstar.argtypes = [ctypes.c_int64, _f64p, _f64p]
        L.oracle_cstar.restype = ctypes.c_double
        L.oracle_draft_rows.argtypes = [ctypes.c_int64, ctypes.c_int64, _f64p, ctypes.c_uint64,
                                        _i32p, _i32p, _i32p, _f64p, _f64p, _f64p]
        L.oracle_verify_requests.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                             _f64p, _f64p, _i32p, _i32p, ctypes.c_uint64, _i32p,
                                             _f32p, _i32p, _i32p, _u8p, _f64p, _f64p, _f64p,
                                             _f64p]
        L.oracle_confidence_rows.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                             _f64p, _f64p, _f64p, _f64p, _f32p]
        L.oracle_prefix_products.argtypes = [ctypes.c_int64, ctypes.c_int64, _f32p, _f32p]
        L.oracle_tau_units.argtypes = [ctypes.c_float]
        L.oracle_tau_units.restype = ctypes.c_int64
        L.oracle_schedule.argtypes = [ctypes.c_int64, ctypes.c_int64, _f32p, _f32p,
                                      ctypes.c_int64, _i32p, _f64p, _f64p, _f64p]
        L.oracle_schedule.restype = ctypes.c_int64
        L.oracle_schedule_capacity.argtypes = [ctypes.c_int64, ctypes.c_int64, _f32p, _f32p,
                                               ctypes.c_int64, _f64p, _f64p]
        L.oracle_schedule_capacity.restype = ctypes.c_int64
        L.oracle_schedule_topk.argtypes = [ctypes.c_int64, ctypes.c_int64, _f32p, _f32p,
                                           ctypes.c_int64, ctypes.c_int64, _i32p, _f64p]
        L.oracle_schedule_topk.restype = ctypes.c_int64
        L.oracle_threshold_lengths.argtypes = [ctypes.c_int64, ctypes.c_int64, _f32p,
                                               ctypes.c_double, _i32p]
        L.oracle_conditional_acceptance.argtypes = [ctypes.c_int64, ctypes.c_int64, _u8p,
                                                    _i64p, _i64p]
        L.oracle_ece_units.argtypes = [ctypes.c_int64, _f32p, _u8p, ctypes.c_int64]
        L.oracle_ece_units.restype = ctypes.c_int64
        L.oracle_sts_fit.argtypes = [ctypes.c_int64, ctypes.c_int64, _f64p, _u8p, ctypes.c_int64,
                                     _f64p, ctypes.c_int64, _f32p, _i64p, _i64p, _f32p]
        L.oracle_threshold_sweep.argtypes = [ctypes.c_int64, ctypes.c_int64, _f32p, _i32p,
                                             ctypes.c_int64, _f64p, _i64p, _i64p]
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def set_threads(n: int):
    """Threads of the oracle's OpenMP row loops."""
    lib().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def _p(a: np.ndarray, ptype):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ptype)


# ---------------------------------------------------------------------------
# stored values -> fp64
# ---------------------------------------------------------------------------
def to_f64(a: np.ndarray) -> np.ndarray:
    """Exact fp64 image of stored tensor values: uint16 arrays hold bfloat16
    bit patterns, float32 arrays hold binary32 values."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    if a.dtype == np.float64:
        return a
    raise TypeError(f"unsupported stored dtype {a.dtype}")


# ---------------------------------------------------------------------------
# random numbers (exposed for the pins)
# ---------------------------------------------------------------------------
def philox(key0: int, key1: int, counter) -> np.ndarray:
    ctr = np.ascontiguousarray(np.asarray(counter, dtype=np.uint32))
    out = np.zeros(4, dtype=np.uint32)
    lib().oracle_philox4x32_10(key0, key1, _p(ctr, _u32p), _p(out, _u32p))
    return out


def word(seed: int, stream: int, r: int, k: int, v: int) -> int:
    return int(lib().oracle_word(seed, stream, r, k, v))


def words(seed: int, stream: int, r: int, k: int, v0: int, n: int) -> np.ndarray:
    out = np.zeros(n, np.uint32)
    lib().oracle_words(seed, stream, r, k, v0, n, _p(out, _u32p))
    return out


def uniform(w: int) -> float:
    return float(lib().oracle_uniform(w))


def gumbel(w: int) -> float:
    return float(lib().oracle_gumbel(w))


# ---------------------------------------------------------------------------
# row primitives (exposed for the pins)
# ---------------------------------------------------------------------------
def logsumexp(z) -> float:
    z = np.ascontiguousarray(z, dtype=np.float64)
    return float(lib().oracle_logsumexp(z.size, _p(z, _f64p)))


def gumbel_argmax(w, g):
    w = np.ascontiguousarray(w, dtype=np.float64)
    g = np.ascontiguousarray(g, dtype=np.float64)
    m = ctypes.c_double()
    idx = lib().oracle_gumbel_argmax(w.size, _p(w, _f64p), _p(g, _f64p), ctypes.byref(m))
    return int(idx), float(m.value)


def two_level_draw(w, block: int, seed: int, stream_block: int, stream_member: int,
                   r: int, k: int):
    """Two-level Gumbel-max draw from softmax(w): returns (index, margin)."""
    w = np.ascontiguousarray(w, dtype=np.float64)
    m = ctypes.c_double()
    idx = lib().oracle_two_level_draw(w.size, _p(w, _f64p), block, seed, stream_block,
                                      stream_member, r, k, ctypes.byref(m))
    return int(idx), float(m.value)


def accept(ln_u: float, lpt_x: float, lpd_x: float) -> bool:
    return bool(lib().oracle_accept(ln_u, lpt_x, lpd_x))


def residual_logw(lpd, lpt):
    lpd = np.ascontiguousarray(lpd, dtype=np.float64)
    lpt = np.ascontiguousarray(lpt, dtype=np.float64)
    out = np.empty_like(lpd)
    npos = lib().oracle_residual_logw(lpd.size, _p(lpd, _f64p), _p(lpt, _f64p), _p(out, _f64p))
    return out, int(npos)


def cstar(lpd, lpt) -> float:
    lpd = np.ascontiguousarray(lpd, dtype=np.float64)
    lpt = np.ascontiguousarray(lpt, dtype=np.float64)
    return float(lib().oracle_cstar(lpd.size, _p(lpd, _f64p), _p(lpt, _f64p)))


# ---------------------------------------------------------------------------
# stage 1: draft  [P1 §3.1; P2 "최종 분포"]
# ---------------------------------------------------------------------------
def draft_logits(U_k: np.ndarray, W1: np.ndarray, W2f: np.ndarray, prev: np.ndarray) -> np.ndarray:
    """z = U_k + W1[prev] @ W2 in fp64 for a set of rows.

    U_k: [n, V] stored values; W1: [V, rank] stored values; W2f: [rank, V] fp64;
    prev: [n] previous tokens (anchors at k = 1)."""
    return to_f64(U_k) + to_f64(W1[prev]) @ W2f


def draft(U, W1, W2, anchors, seed: int, requests=None):
    """Draft all gamma positions for the given requests (default: all).

    Returns dict with tokens [n, gamma] int32, lse, logq, margin [n, gamma] fp64,
    for the requests in ``requests`` order."""
    R, gamma, V = U.shape
    req = np.arange(R, dtype=np.int32) if requests is None else np.asarray(requests, np.int32)
    n = req.size
    W2f = to_f64(W2)
    tokens = np.zeros((n, gamma), np.int32)
    lse = np.zeros((n, gamma), np.float64)
    logq = np.zeros((n, gamma), np.float64)
    margin = np.zeros((n, gamma), np.float64)
    prev = np.asarray(anchors, np.int32)[req].copy()
    for k in range(1, gamma + 1):
        z = np.ascontiguousarray(draft_logits(U[req, k - 1, :], W1, W2f, prev))
        kk = np.full(n, k, np.int32)
        t = np.zeros(n, np.int32)
        l = np.zeros(n, np.float64)
        q = np.zeros(n, np.float64)
        m = np.zeros(n, np.float64)
        lib().oracle_draft_rows(n, V, _p(z, _f64p), seed, _p(req, _i32p), _p(kk, _i32p),
                                _p(t, _i32p), _p(l, _f64p), _p(q, _f64p), _p(m, _f64p))
        tokens[:, k - 1] = t
        lse[:, k - 1] = l
        logq[:, k - 1] = q
        margin[:, k - 1] = m
        prev = t
    return {"requests": req, "tokens": tokens, "lse": lse, "logq": logq, "margin": margin}


def draft_logits_all(U, W1, W2f, anchors_req, tokens_req, req) -> np.ndarray:
    """Draft logits of every position for the given requests: [n, gamma, V] fp64."""
    R, gamma, V = U.shape
    n = len(req)
    out = np.empty((n, gamma, V), np.float64)
    for k in range(1, gamma + 1):
        prev = anchors_req if k == 1 else tokens_req[:, k - 2]
        out[:, k - 1, :] = draft_logits(U[req, k - 1, :], W1, W2f, prev)
    return out


# ---------------------------------------------------------------------------
# stage 2: verify  [P1 요약, §3.2.1; P2 배경]
# ---------------------------------------------------------------------------
def verify(U, W1, W2, anchors, tokens, T, lengths, seed: int, requests=None, chunk: int = 8):
    """Verify the given requests.  tokens: [R, gamma] (full batch, indexed by
    request id), T: [R, gamma+1, V] stored target logits, lengths: [R] or None
    (all gamma).  Returns per-request arrays in ``requests`` order."""
    R, gamma, V = U.shape
    req = np.arange(R, dtype=np.int32) if requests is None else np.asarray(requests, np.int32)
    lengths = np.full(R, gamma, np.int32) if lengths is None else np.asarray(lengths, np.int32)
    anchors = np.asarray(anchors, np.int32)
    tokens = np.asarray(tokens, np.int32)
    W2f = to_f64(W2)
    n = req.size
    out = {
        "requests": req,
        "cstar": np.zeros((n, gamma), np.float32),
        "n_accept": np.zeros(n, np.int32),
        "out_token": np.zeros(n, np.int32),
        "accept_mask": np.zeros((n, gamma), np.uint8),
        "acc_margin": np.zeros((n, gamma), np.float64),
        "out_margin": np.zeros(n, np.float64),
        "lse_t": np.zeros((n, gamma + 1), np.float64),
        "lse_d": np.zeros((n, gamma), np.float64),
    }
    for c0 in range(0, n, chunk):
        rq = np.ascontiguousarray(req[c0:c0 + chunk])
        m = rq.size
        zd = np.ascontiguousarray(draft_logits_all(U, W1, W2f, anchors[rq], tokens[rq], rq))
        zt = np.ascontiguousarray(to_f64(T[rq]))
        tk = np.ascontiguousarray(tokens[rq])
        ln = np.ascontiguousarray(lengths[rq])
        cs = np.zeros((m, gamma), np.float32)
        na = np.zeros(m, np.int32)
        ot = np.zeros(m, np.int32)
        am = np.zeros((m, gamma), np.uint8)
        acm = np.zeros((m, gamma), np.float64)
        om = np.zeros(m, np.float64)
        lt = np.zeros((m, gamma + 1), np.float64)
        ld = np.zeros((m, gamma), np.float64)
        lib().oracle_verify_requests(m, gamma, V, _p(zd, _f64p), _p(zt, _f64p), _p(tk, _i32p),
                                     _p(ln, _i32p), seed, _p(rq, _i32p), _p(cs, _f32p),
                                     _p(na, _i32p), _p(ot, _i32p), _p(am, _u8p), _p(acm, _f64p),
                                     _p(om, _f64p), _p(lt, _f64p), _p(ld, _f64p))
        sl = slice(c0, c0 + m)
        out["cstar"][sl] = cs
        out["n_accept"][sl] = na
        out["out_token"][sl] = ot
        out["accept_mask"][sl] = am
        out["acc_margin"][sl] = acm
        out["out_margin"][sl] = om
        out["lse_t"][sl] = lt
        out["lse_d"][sl] = ld
    return out


# ---------------------------------------------------------------------------
# confidence head + STS  [P1 §3.2.1]
# ---------------------------------------------------------------------------
def confidence(h, w, temps, W1, anchors, tokens, requests=None):
    """c[r,k] = sigmoid((w . [h_{r,k}; W1[x_{r,k-1}]]) / T_k) for the given requests."""
    R, gamma, H = h.shape
    rank = W1.shape[1]
    req = np.arange(R, dtype=np.int32) if requests is None else np.asarray(requests, np.int32)
    anchors = np.asarray(anchors, np.int32)
    tokens = np.asarray(tokens, np.int32)
    prev = np.concatenate([anchors[req, None], tokens[req, :gamma - 1]], axis=1)  # [n, gamma]
    hf = np.ascontiguousarray(to_f64(h[req]).reshape(-1, H))
    ef = np.ascontiguousarray(to_f64(W1[prev.reshape(-1)]))
    wf = np.ascontiguousarray(np.asarray(w, np.float64))
    tf = np.ascontiguousarray(np.tile(np.asarray(temps, np.float64), req.size))
    c = np.zeros(req.size * gamma, np.float32)
    lib().oracle_confidence_rows(req.size * gamma, H, rank, _p(hf, _f64p), _p(ef, _f64p),
                                 _p(wf, _f64p), _p(tf, _f64p), _p(c, _f32p))
    return c.reshape(req.size, gamma)


# ---------------------------------------------------------------------------
# stages 3-4: prefix products and Algorithm 1  [P1 §3.2.2]
# ---------------------------------------------------------------------------
def prefix_products(c: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.float32)
    R, gamma = c.shape
    a = np.zeros_like(c)
    lib().oracle_prefix_products(R, gamma, _p(c, _f32p), _p(a, _f32p))
    return a


def tau_units(a: float) -> int:
    return int(lib().oracle_tau_units(ctypes.c_float(a)))


def schedule(a: np.ndarray, sps: np.ndarray):
    """Algorithm 1 on prefix products a [R, gamma]; returns dict with lengths,
    stats (B, tau, Theta, n_sel), theta_path [R*gamma+1] and stop_gap."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    sps = np.ascontiguousarray(sps, dtype=np.float32)
    R, gamma = a.shape
    lengths = np.zeros(R, np.int32)
    stats = np.zeros(4, np.float64)
    path = np.full(R * gamma + 1, np.nan)
    gap = ctypes.c_double()
    sel = lib().oracle_schedule(R, gamma, _p(a, _f32p), _p(sps, _f32p), sps.size,
                                _p(lengths, _i32p), _p(stats, _f64p), _p(path, _f64p),
                                ctypes.byref(gap))
    if sel < 0:
        raise ValueError("SPS table shorter than R*(gamma+1)")
    return {"lengths": lengths, "stats": stats, "theta_path": path, "stop_gap": gap.value,
            "n_sel": int(sel)}


# ---------------------------------------------------------------------------
# production scheduler: capacity from past rounds, top-K now  [P1 §5.2]
# ---------------------------------------------------------------------------
def schedule_capacity(a: np.ndarray, sps: np.ndarray):
    """Capacity K: the candidate count (survival order) with the largest Theta
    along the whole path, no early stop; returns dict K, stats, theta_path."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    sps = np.ascontiguousarray(sps, dtype=np.float32)
    R, gamma = a.shape
    stats = np.zeros(4, np.float64)
    path = np.full(R * gamma + 1, np.nan)
    K = lib().oracle_schedule_capacity(R, gamma, _p(a, _f32p), _p(sps, _f32p), sps.size,
                                       _p(stats, _f64p), _p(path, _f64p))
    if K < 0:
        raise ValueError("SPS table shorter than R*(gamma+1)")
    return {"K": int(K), "stats": stats, "theta_path": path}


def schedule_topk(a: np.ndarray, sps: np.ndarray, K: int):
    """Verify the first min(K, R*gamma) candidates in survival order."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    sps = np.ascontiguousarray(sps, dtype=np.float32)
    R, gamma = a.shape
    lengths = np.zeros(R, np.int32)
    stats = np.zeros(4, np.float64)
    t = lib().oracle_schedule_topk(R, gamma, _p(a, _f32p), _p(sps, _f32p), sps.size, int(K),
                                   _p(lengths, _i32p), _p(stats, _f64p))
    if t < 0:
        raise ValueError("SPS table shorter than R*(gamma+1), or K < 0")
    return {"lengths": lengths, "stats": stats}


# ---------------------------------------------------------------------------
# static threshold, conditional acceptance, threshold sweep  [P1 §4.3.1, §4.3.3]
# ---------------------------------------------------------------------------
def threshold_lengths(a: np.ndarray, theta: float) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    R, gamma = a.shape
    lengths = np.zeros(R, np.int32)
    lib().oracle_threshold_lengths(R, gamma, _p(a, _f32p), float(theta), _p(lengths, _i32p))
    return lengths


def conditional_acceptance(mask: np.ndarray):
    """(reached[k], accepted[k]) per position from an accept mask [R, gamma]."""
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    R, gamma = mask.shape
    reached = np.zeros(gamma, np.int64)
    accepted = np.zeros(gamma, np.int64)
    lib().oracle_conditional_acceptance(R, gamma, _p(mask, _u8p), _p(reached, _i64p),
                                        _p(accepted, _i64p))
    return reached, accepted


def threshold_sweep(a: np.ndarray, n_accept: np.ndarray, thresholds):
    """(verified[g], accepted[g]) for each threshold of a fully verified round."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    na = np.ascontiguousarray(n_accept, dtype=np.int32)
    th = np.ascontiguousarray(thresholds, dtype=np.float64)
    R, gamma = a.shape
    ver = np.zeros(th.size, np.int64)
    acc = np.zeros(th.size, np.int64)
    lib().oracle_threshold_sweep(R, gamma, _p(a, _f32p), _p(na, _i32p), th.size, _p(th, _f64p),
                                 _p(ver, _i64p), _p(acc, _i64p))
    return ver, acc


# ---------------------------------------------------------------------------
# Sequential Temperature Scaling fit  [P1 §3.2.1]
# ---------------------------------------------------------------------------
#: ECE sums are exact integers in units of 2^-40 of survival probability
ECE_UNIT = 2.0 ** -40


def ece_units(a: np.ndarray, y: np.ndarray, bins: int) -> int:
    """N * ECE of survival values a [N] against 0/1 labels y [N], in ECE_UNIT."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    y = np.ascontiguousarray(y, dtype=np.uint8)
    return int(lib().oracle_ece_units(a.size, _p(a, _f32p), _p(y, _u8p), int(bins)))


def sts_fit(s: np.ndarray, y: np.ndarray, grid, bins: int = 15):
    """Left-to-right temperature grid search.  s [N, gamma] scores, y [N, gamma]
    survival labels, grid [G] candidate temperatures.  Returns temps [gamma],
    ece [gamma] and ece_at_1 [gamma] (as fractions: units * ECE_UNIT / N), the
    integer unit values, and the calibrated survival a [N, gamma]."""
    s = np.ascontiguousarray(s, dtype=np.float64)
    y = np.ascontiguousarray(y, dtype=np.uint8)
    grid = np.ascontiguousarray(grid, dtype=np.float64)
    N, gamma = s.shape
    temps = np.zeros(gamma, np.float32)
    eu = np.zeros(gamma, np.int64)
    e1 = np.zeros(gamma, np.int64)
    a = np.zeros((N, gamma), np.float32)
    lib().oracle_sts_fit(N, gamma, _p(s, _f64p), _p(y, _u8p), grid.size, _p(grid, _f64p), int(bins),
                         _p(temps, _f32p), _p(eu, _i64p), _p(e1, _i64p), _p(a, _f32p))
    return {"temps": temps, "ece_units": eu, "ece1_units": e1,
            "ece": eu * ECE_UNIT / max(N, 1), "ece_at_1": e1 * ECE_UNIT / max(N, 1), "a": a}


# ---------------------------------------------------------------------------
# multi-round decoding  [P1 §요약, §3, §3.1]
# ---------------------------------------------------------------------------
def round_key(seed: int, t: int) -> int:
    """READING: round t draws with the Philox key seed + t * 2^32 (mod 2^64)."""
    return (int(seed) + (int(t) << 32)) % (1 << 64)


def decode_rounds(W1, W2, anchors, seed: int, rounds: int, backbone, target):
    """Rounds of draft + verify of every position: round t drafts from the
    anchors with U = backbone(t), takes T = target(t, U, anchors, tokens) and emits the
    accepted prefix plus the corrective or bonus token, which is the next
    round's anchor.  Returns one dict per round (draft and verify outputs, the
    round's anchors and key)."""
    out = []
    anchors = np.asarray(anchors, np.int32).copy()
    for t in range(rounds):
        key = round_key(seed, t)
        U = backbone(t)
        d = draft(U, W1, W2, anchors, key)
        T = target(t, U, anchors, d["tokens"])
        v = verify(U, W1, W2, anchors, d["tokens"], T, None, key)
        out.append({"anchors": anchors.copy(), "key": key, "U": U, "T": T, "draft": d,
                    "verify": v})
        anchors = v["out_token"].astype(np.int32).copy()
    return out
